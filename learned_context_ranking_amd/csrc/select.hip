// Gate normalisation and Top-K block selection, one wavefront per score row.
//
// [SAS-ko] "무엇과 다른가", choice 2: g = softmax(s) over the row's valid history blocks,
// log g_m = s_m - LSE(s). [SAS-ja] "前提" / "仕組み" (Algorithm 2): the K best-scoring
// history blocks are attended. Selection compares the fp32 scores themselves; ties go to
// the lower block index, -0 equals +0 and NaN ranks as -inf.
//
// Each lane holds PL scores (element m = lane + 64 i, so loads are coalesced); only the
// registers that hold valid scores of the row take part (rows of a prefill have j valid
// scores). The K-th largest order-preserving key is found by fixing its 32 bits from the
// top (topk_cut): a candidate bit stays set when at least K keys are >= the candidate; the
// search stops as soon as a candidate admits exactly K keys (they are the kept set).
// Otherwise blocks strictly above the threshold are kept and, among the blocks equal to it,
// the lowest indices fill the remaining places. A ballot prefix count (topk_walk) writes
// the kept indices in ascending order without any sort.
#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

// log g of a kept block with score x (NaN already read as -inf) under each activation;
// norm is the softmax normaliser (LSE over the history or over the kept set)
__device__ __forceinline__ float log_gate(int gate, float x, float norm) {
  if (gate == kGateSigmoid) {
    // log sigmoid(x) = min(x, 0) - log(1 + e^-|x|)
    return x == -INFINITY ? -INFINITY : fminf(x, 0.0f) - log1pf(expf(-fabsf(x)));
  }
  if (gate == kGateExp) return x;
  return norm == -INFINITY ? -INFINITY : x - norm;
}

// GATE: the activation whose log g is written (a compile-time choice, so each launch
// carries only its own code path: the per-register walks below are fully unrolled)
constexpr int kStageCap = 256;   // rows with kcap up to this stage their output in LDS

// One wave's row with its valid scores in the first NR registers of each lane (NR is the
// smallest quarter step of PL that holds them): loads, LSE, search and walk run over NR
// registers only, so the short rows of a prefill (row j has j valid scores) do not pay
// for the longest. PL is the register count of the widest row (the gate output is
// written over all of it).
template <int NR, int PL, int GATE>
__device__ __forceinline__ void select_row(const SelectArgs& a, long long row, int valid, int* s_idx,
                                           float* s_lg) {
  const int lane = threadIdx.x & 63;
  const float* srow = a.s + row * a.ld;

  // Loads without branches (the index clamped into the valid columns, which are the only
  // ones read), so all NR loads are in flight together; masks are applied afterwards.
  float x[NR];
  if (valid > 0) {
#pragma unroll
    for (int i = 0; i < NR; ++i) x[i] = srow[min(lane + 64 * i, valid - 1)];
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float v = valid > 0 ? x[i] : -INFINITY;
    v = (lane + 64 * i < valid && v == v) ? v : -INFINITY;   // NaN ranks as -inf
    x[i] = v == 0.0f ? 0.0f : v;                             // -0 -> +0
  }

  // LSE over the valid scores.
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NR; ++i) mx = fmaxf(mx, x[i]);
  mx = dpp_max(mx);
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    // sum of e^(x - mx) as 2^((x - mx) log2 e) on the hardware exp2 (one instruction, where
    // expf's full-range version takes about a dozen): every term is <= 1, the largest is
    // 1, and a term the hardware flushes (below 2^-126) changes no fp32 sum that holds it
    const float mxl = mx * kLog2e;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NR; ++i) sum += __builtin_amdgcn_exp2f(fmaf(x[i], kLog2e, -mxl));
    sum = dpp_sum(sum);
    lse = mx + logf(sum);
  }
  if (a.lse != nullptr && lane == 0 && (!a.do_select || GATE == kGateSoftmax)) a.lse[row] = lse;
  if (a.g != nullptr) {
    float* grow = a.g + row * a.ld;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int m = lane + 64 * i;
      if (m < a.cols) grow[m] = (i < NR && m < valid && lse != -INFINITY) ? expf(x[i < NR ? i : 0] - lse) : 0.0f;
    }
  }
  if (!a.do_select) return;

  const int k = a.full ? valid : min(a.topk, valid);
  int32_t* idx_row = a.idx + row * a.kcap;
  float* lg_row = a.logg != nullptr ? a.logg + row * a.kcap : nullptr;
  if (k > 0) {
    const int nreg = (valid + 63) >> 6;   // registers holding valid scores (uniform)
    uint32_t key[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) key[i] = (lane + 64 * i < valid) ? order_key(x[i]) : 0u;
    uint32_t T;
    int need_eq;
    topk_cut(key, nreg, valid, k, T, need_eq);
    auto walk = [&](auto&& f) { topk_walk(key, nreg, T, need_eq, f); };
    // The walks take each kept score back from its key (exact), so that x[] is no longer
    // live: that leaves the widest rows registers to spare.
    float norm = lse;   // the gate's normaliser (reported as lse)
    if (GATE == kGateSoftmaxSelected) {
      float m = -INFINITY, sum = 0.0f;   // online LSE over the kept scores
      walk([&](int i, int) {
        const float xi = key_score(key[i]);
        if (xi > m) { sum = sum * expf(m - xi) + 1.0f; m = xi; }
        else if (xi != -INFINITY) sum += expf(xi - m);
      });
      const float wm = dpp_max(m);
      sum = dpp_sum(m == -INFINITY ? 0.0f : sum * expf(m - wm));
      norm = wm == -INFINITY ? -INFINITY : wm + logf(sum);
    } else if (GATE != kGateSoftmax) {
      norm = 0.0f;
    }
    if (a.lse != nullptr && lane == 0 && GATE != kGateSoftmax) a.lse[row] = norm;
    if (a.kcap <= kStageCap) {
      // a row's kept entries are few per register (one or two lanes): gather them in LDS
      walk([&](int i, int pos) {
        s_idx[pos] = lane + 64 * i;
        s_lg[pos] = log_gate(GATE, key_score(key[i]), norm);
      });
    } else {
      walk([&](int i, int pos) {
        idx_row[pos] = lane + 64 * i;
        if (lg_row != nullptr) lg_row[pos] = log_gate(GATE, key_score(key[i]), norm);
      });
    }
  } else if (a.lse != nullptr && lane == 0 && GATE != kGateSoftmax) {
    a.lse[row] = GATE == kGateSoftmaxSelected ? -INFINITY : 0.0f;
  }
  if (a.kcap <= kStageCap) {
    // the row's LDS entries were written by this wave's own lanes: make them visible to
    // the other lanes (LDS accesses of one wave complete in order once issued)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int p = lane; p < a.kcap; p += 64) {
      const bool kept = p < k;
      idx_row[p] = kept ? s_idx[p] : -1;
      if (lg_row != nullptr) lg_row[p] = kept ? s_lg[p] : 0.0f;
    }
  } else {
    for (int p = k + lane; p < a.kcap; p += 64) {
      idx_row[p] = -1;
      if (lg_row != nullptr) lg_row[p] = 0.0f;
    }
  }
  if (lane == 0) a.cnt[row] = k;
}

template <int PL, int GATE>
__global__ __launch_bounds__(256) void select_kernel(const SelectArgs a) {
  // kept (index, log g) of each wave's row, written out with coalesced stores at the end
  __shared__ int s_idx[4][kStageCap];
  __shared__ float s_lg[4][kStageCap];
  const int wv = threadIdx.x >> 6;
  // Rows in reverse order: a prefill's rows grow with j within each (batch, head), so the
  // longest rows start early and the launch ends on short ones.
  const long long row = a.R - 1 - ((long long)blockIdx.x * 4 + (threadIdx.x >> 6));
  if (row < 0) return;  // uniform per wave
  int valid;
  if (a.mode == 0) {
    valid = (int)(row % a.rows);
  } else {
    const long long b = row / ((long long)a.H * a.rows);
    valid = a.row_valid[b];
  }
  valid = __builtin_amdgcn_readfirstlane(min(max(valid, 0), a.cols));
  const int nreg = (valid + 63) >> 6;
  if constexpr (PL >= 4) {
    if (nreg <= PL / 4) select_row<PL / 4, PL, GATE>(a, row, valid, s_idx[wv], s_lg[wv]);
    else if (nreg <= PL / 2) select_row<PL / 2, PL, GATE>(a, row, valid, s_idx[wv], s_lg[wv]);
    else if (nreg <= 3 * PL / 4) select_row<3 * PL / 4, PL, GATE>(a, row, valid, s_idx[wv], s_lg[wv]);
    else select_row<PL, PL, GATE>(a, row, valid, s_idx[wv], s_lg[wv]);
  } else {
    select_row<PL, PL, GATE>(a, row, valid, s_idx[wv], s_lg[wv]);
  }
}

template <int PL>
static void launch_select_pl(const SelectArgs& a, dim3 grid, dim3 block, hipStream_t st) {
  const int gate = a.do_select ? a.gate : kGateSoftmax;   // gates only: the softmax normaliser
  if (gate == kGateSoftmaxSelected) hipLaunchKernelGGL((select_kernel<PL, kGateSoftmaxSelected>), grid, block, 0, st, a);
  else if (gate == kGateSigmoid) hipLaunchKernelGGL((select_kernel<PL, kGateSigmoid>), grid, block, 0, st, a);
  else if (gate == kGateExp) hipLaunchKernelGGL((select_kernel<PL, kGateExp>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((select_kernel<PL, kGateSoftmax>), grid, block, 0, st, a);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.R + 3) / 4)), block(256);
  const int c = a.cols;
  ProfScope prof("select", st);
  if (c <= 64) launch_select_pl<1>(a, grid, block, st);
  else if (c <= 128) launch_select_pl<2>(a, grid, block, st);
  else if (c <= 256) launch_select_pl<4>(a, grid, block, st);
  else if (c <= 512) launch_select_pl<8>(a, grid, block, st);
  else if (c <= 1024) launch_select_pl<16>(a, grid, block, st);
  else if (c <= 2048) launch_select_pl<32>(a, grid, block, st);
  else if (c <= 4096) launch_select_pl<64>(a, grid, block, st);
  else launch_select_pl<128>(a, grid, block, st);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gate softmax backward

// [SAS-ko] "무엇과 다른가", choice 2 (g = softmax(s) over the valid history) with choice 4
// (sparse scope: only selected blocks have a gradient dL/dg of their own): the chain rule
// through the softmax gives ds_m = g_m (dg_m - c), c = sum over the selected slots of
// g dg, for every valid m (dg_m = 0 when m is not selected). One wavefront per score row;
// the selected blocks are marked in an LDS bitmap so every ds entry is written once.
__global__ __launch_bounds__(256) void gates_bwd_kernel(const GatesBwdArgs a) {
  __shared__ uint32_t sel_bits[4][kMaxCols / 32];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + w;
  const bool live = row < a.R;
  int valid = 0;
  if (live) {
    if (a.mode == 0) {
      valid = (int)(row % a.rows);
    } else {
      const long long b = row / ((long long)a.H * a.rows);
      valid = a.row_valid[b];
    }
    valid = min(max(valid, 0), a.cols);
  }
  const float* srow = a.s + row * a.ld;
  float* drow = a.ds + row * a.ld;
  const float lse = (live && a.lse != nullptr) ? a.lse[row] : -INFINITY;
  const float lse2 = lse * kLog2e;
  const int cnt = live ? min(max(a.cnt[row], 0), a.kcap) : 0;
  const int32_t* irow = a.idx + row * a.kcap;
  const float* grow = a.dg + row * a.kcap;
  // gate of block m (0 for a NaN or -inf score, or a row without finite LSE)
  auto gate = [&](int m) {
    const float v = srow[m];
    if (!(v > -INFINITY)) return 0.0f;   // -inf or NaN score: gate 0
    if (a.gate == kGateSigmoid) return 1.0f / (1.0f + expf(-v));
    if (a.gate == kGateExp) return expf(v);
    if (!(lse > -INFINITY)) return 0.0f;
    return __builtin_amdgcn_exp2f(fmaf(v, kLog2e, -lse2));   // e^(v - lse) <= 1 on the hardware exp2
  };
  const bool softmax_like = a.gate == kGateSoftmax || a.gate == kGateSoftmaxSelected;
  for (int i = lane; i < kMaxCols / 32; i += 64) sel_bits[w][i] = 0u;
  __syncthreads();
  float c = 0.0f;
  for (int t = lane; t < cnt; t += 64) {
    const int m = irow[t];
    if (m >= 0 && m < valid) {
      atomicOr(&sel_bits[w][m >> 5], 1u << (m & 31));
      if (softmax_like) c += gate(m) * grow[t];
    }
  }
  c = dpp_sum(c);
  __syncthreads();
  if (!live) return;  // uniform per wave; no barrier follows
  for (int m = lane; m < a.ld; m += 64) {
    if (m >= valid) {
      drow[m] = 0.0f;
    } else if (!((sel_bits[w][m >> 5] >> (m & 31)) & 1u)) {
      // only the history softmax couples unselected blocks to the kept ones
      drow[m] = a.gate == kGateSoftmax ? -gate(m) * c : 0.0f;
    }
  }
  for (int t = lane; t < cnt; t += 64) {
    const int m = irow[t];
    if (m >= 0 && m < valid) {
      const float g = gate(m);
      drow[m] = softmax_like ? g * (grow[t] - c) : (a.gate == kGateSigmoid ? grow[t] * g * (1.0f - g) : grow[t] * g);
    }
  }
}

hipError_t launch_gates_bwd(const GatesBwdArgs& a, hipStream_t st) {
  ProfScope prof("gates_bwd", st);
  hipLaunchKernelGGL(gates_bwd_kernel, dim3((unsigned)((a.R + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sas
