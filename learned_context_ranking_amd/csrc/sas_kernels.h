// Internal launch interface between the C ABI host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sas {

// Brackets one kernel launch with HIP events on its stream while timing is enabled
// (sas_profile_enable); does nothing otherwise.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t st);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t st_;
  void* a_;
};

// Order in which a launch's workgroups take their work items (a debugging aid, see
// sas_debug_workgroup_order): work item = (blockIdx.x * mul + add) mod gridDim.x, a
// bijection when mul and the grid size are coprime. The natural order is mul = 1, add = 0.
struct WgOrder {
  uint32_t mul = 1, add = 0;
};
// the order for a launch of `grid` workgroups under the library's current debug seed
WgOrder wg_order(unsigned grid);
__device__ __forceinline__ unsigned wg_index(WgOrder o) {
  return (unsigned)(((unsigned long long)blockIdx.x * o.mul + o.add) % gridDim.x);
}

// gate activations (sas_gate in include/sas.h)
constexpr int kGateSoftmax = 0, kGateSoftmaxSelected = 1, kGateSigmoid = 2, kGateExp = 3;

struct SelectArgs {
  const float* s;
  long long R;          // rows in total = B * H * rows
  int H, rows, cols;
  long long ld;
  int mode;             // 0 prefill, 1 decode
  const int32_t* row_valid;
  int topk, full, kcap, do_select, gate;
  int32_t* idx;
  int32_t* cnt;
  float* lse;
  float* logg;
  float* g;
};
hipError_t launch_select(const SelectArgs& a, hipStream_t st);

constexpr int kMaxCols = 8192;   // longest score row (history blocks) the selection handles

struct GatesBwdArgs {
  const float* s;
  long long R;          // rows in total = B * H * rows
  int H, rows, cols;
  long long ld;
  int mode;             // 0 prefill, 1 decode
  const int32_t* row_valid;
  const float* lse;
  const int32_t* idx;
  const int32_t* cnt;
  const float* dg;
  int kcap;
  int gate;
  float* ds;
};
hipError_t launch_gates_bwd(const GatesBwdArgs& a, hipStream_t st);

struct PoolArgs {
  const uint16_t* K;    // [B][Hkv][Lmax][d] bf16, or with page_table a pool [num_pages][Hkv][64][d]
  int B, Hkv, Lmax, C, d;
  const int32_t* kv_len;
  int first_block, nblk;   // blocks first_block .. first_block + nblk - 1
  uint16_t* kbar;       // [B][Hkv][C][d] bf16
  // paged cache (page_table != null): block m of sequence b is page page_table[b * C + m];
  // a page id outside [0, num_pages) pools to zero
  const int32_t* page_table;
  int num_pages;
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t st);

struct DecSelArgs {
  const uint16_t* q;    // [B][Hq][d] bf16
  const uint16_t* kbar; // [B][Hkv][C][d] bf16
  int B, Hq, Hkv, G, d, C;
  const int32_t* kv_len;
  float scale;
  int topk, kcap;
  float* s;             // [B][Hkv][C]
  int32_t* idx;         // [B][Hkv][kcap]
  int32_t* cnt;         // [B][Hkv]
  float* lse;           // [B][Hkv] or null
  float* logg;          // [B][Hkv][kcap] or null
  // candidates (launch_decode_candidates): per chunk of cch blocks its min(topk, blocks)
  // best, as (score, block) in topk slots, ascending block, empty slots block -1;
  // cs / ci are [B][Hkv][cld], cld = ceil(C / cch) * topk
  float* cs;
  int32_t* ci;
  int cch, cld;
  int hist_cap;         // (candidates) history blocks of a row at most: the decode's, (Lmax - 1) / 64
};
hipError_t launch_decode_select(const DecSelArgs& a, hipStream_t st);
// Candidate chunk size in blocks for rows of C blocks and K = topk: the smallest
// (4 waves x blocks per wave) x 2^r that leaves at most kDecSelMaxCols slots per row.
int decode_cand_chunk(int C, int topk, int d);
hipError_t launch_decode_candidates(const DecSelArgs& a, hipStream_t st);

struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  const uint16_t* O;     // backward only
  const uint16_t* dO;    // backward only
  const int32_t* idx;
  const int32_t* cnt;
  const float* logg;     // may be null
  int B, Hq, Hkv, n, d, kcap;
  float scale;
  int gate_out;          // 1: gate after the softmax (weights p g), 0: log g inside the logits
  uint16_t* Oout;        // forward output
  float* lse_rows;       // forward output / backward input
  float* dQ;
  float* dK;
  float* dV;
  float* dg;
  // backward workspace pieces
  float* ndelta;         // -delta_t = -dO_t . o_t per query row
  float* nlse;           // -LSE_t / scale per query row (the score offset of the key-major pass)
  float* dg_part;        // [nsplit][rows][kcap] per-split gate-gradient partials
  int32_t* inv_cnt;
  int32_t* inv_off;
  int32_t* inv_list;
  int4* seg_tab;         // key-major work plan: per (b, KV head) NB + dkv_budget segments
  int4* red_tab;         // split key blocks, per (b, KV head) dkv_budget entries
  float* dkv_part;       // partial dK / dV of segments 1.. of split blocks
  int dkv_budget;        // partial slots per (b, KV head)
  WgOrder wg;            // workgroup order of the launch (set by the launcher)
};
hipError_t launch_fwd(const AttnArgs& a, hipStream_t st);
size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int n, int d, int kcap);
hipError_t launch_bwd(AttnArgs a, void* ws, hipStream_t st);

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* Kc;
  const uint16_t* Vc;
  const int32_t* kv_len;
  long long Lmax;
  const int32_t* idx;
  const int32_t* cnt;
  const float* logg;
  int B, Hq, Hkv, d, kcap;
  float scale;
  uint16_t* o;
  float* part;           // workspace: partial (m, l, acc) per chunk
  int bpc;               // blocks per chunk
  int nchunk;            // chunks per (b, h_kv) = ceil((kcap + 1) / bpc)
  // paged cache (page_table != null): Kc / Vc are pools [num_pages][Hkv][64][d], logical
  // block m of sequence b lives in page page_table[b * max_pages + m]; Lmax = 64 max_pages
  const int32_t* page_table;
  int max_pages, num_pages;
  // early stop (order != null): order key of each kept block [B][Hkv][kcap], threshold,
  // blocks used per query head [B][Hq] (nullable)
  const float* order;
  float tau;
  int32_t* used;
  // selection in the same launch (s != null): history scores [B][Hkv][s_ld], K = topk
  // (kcap = topk); the kept blocks written to idx_out [B][Hkv][kcap] / cnt_out [B][Hkv]
  // when idx_out is not null
  const float* s;
  int s_ld, topk;
  int32_t* idx_out;
  int32_t* cnt_out;
  // (candidates) block of each score slot [B][Hkv][s_ld], -1 for an empty slot; slots in
  // ascending block order. With s_id == null slot m is block m.
  const int32_t* s_id;
  WgOrder wg;            // workgroup order of the decode launch (set by the launcher)
};
constexpr int kDecSelMax = 64;        // largest K of the decode with its own selection
constexpr int kDecSelMaxCols = 1024;  // largest number of history blocks it ranks
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int d, int kcap);
// sets a.bpc and a.nchunk as launch_decode will
void decode_plan(DecodeArgs& a);
// bytes of partial states the planned launch writes (0 when every list is one chunk)
size_t decode_part_bytes(const DecodeArgs& a);
hipError_t launch_decode(DecodeArgs a, hipStream_t st);

}  // namespace sas
