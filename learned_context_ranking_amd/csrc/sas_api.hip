// C ABI host layer: argument checks, workspace carving and kernel launches.
// Every check runs before any HIP call, so a rejected call enqueues nothing and touches
// no device state (the checks also run on machines without a GPU).
#include <math.h>
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/sas.h"
#include "sas_kernels.h"

namespace {

thread_local std::string g_last_error;

sas_status fail(sas_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sas_status ok() {
  g_last_error.clear();
  return SAS_OK;
}

sas_status hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE(cond, code, ...)                   \
  do {                                             \
    if (!(cond)) return fail(code, __VA_ARGS__);   \
  } while (0)

sas_status check_rows(const float* s, int B, int H, int rows, int cols, int ld, int mode,
                      const int32_t* row_valid) {
  REQUIRE(s != nullptr, SAS_ERR_INVALID_ARG, "s is NULL");
  REQUIRE(B > 0 && H > 0 && rows > 0, SAS_ERR_INVALID_ARG, "B, H, rows must be > 0 (got %d, %d, %d)", B, H, rows);
  REQUIRE(cols > 0 && cols <= ld, SAS_ERR_INVALID_ARG, "need 0 < cols <= ld (got cols=%d ld=%d)", cols, ld);
  REQUIRE(cols <= 8192, SAS_ERR_UNSUPPORTED, "cols=%d exceeds 8192", cols);
  REQUIRE(mode == SAS_ROWS_PREFILL || mode == SAS_ROWS_DECODE, SAS_ERR_INVALID_ARG, "bad mode %d", mode);
  if (mode == SAS_ROWS_PREFILL) {
    REQUIRE(row_valid == nullptr, SAS_ERR_INVALID_ARG, "row_valid must be NULL in PREFILL mode");
    REQUIRE(cols >= rows - 1, SAS_ERR_INVALID_ARG, "PREFILL needs cols >= rows - 1 (cols=%d rows=%d)", cols, rows);
  } else {
    REQUIRE(row_valid != nullptr, SAS_ERR_INVALID_ARG, "row_valid is required in DECODE mode");
  }
  REQUIRE((long long)B * H * rows < (1ll << 31), SAS_ERR_UNSUPPORTED, "too many rows");
  return SAS_OK;
}

sas_status check_attn(const void* Q, const void* K, const void* V, const int32_t* idx,
                      const int32_t* cnt, const float* logg, int B, int Hq, int Hkv, int n,
                      int d, int block, int kcap, float scale) {
  REQUIRE(Q && K && V, SAS_ERR_INVALID_ARG, "Q, K and V must be non-NULL");
  REQUIRE(cnt != nullptr, SAS_ERR_INVALID_ARG, "cnt is NULL");
  REQUIRE(kcap == 0 || idx != nullptr, SAS_ERR_INVALID_ARG, "idx is NULL");
  REQUIRE(B > 0 && Hq > 0 && Hkv > 0 && n > 0, SAS_ERR_INVALID_ARG, "B, Hq, Hkv, n must be > 0");
  REQUIRE(Hq % Hkv == 0, SAS_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  REQUIRE(block == 64, SAS_ERR_UNSUPPORTED, "block must be 64 (got %d)", block);
  REQUIRE(n % 64 == 0, SAS_ERR_INVALID_ARG, "n=%d is not a multiple of 64", n);
  REQUIRE(d == 64 || d == 128, SAS_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  REQUIRE(kcap >= 0 && kcap <= 8192, SAS_ERR_INVALID_ARG, "kcap=%d out of [0, 8192]", kcap);
  // the backward keeps -LSE / scale per row, finite for every finite LSE when scale >= 1e-30
  REQUIRE(isfinite(scale) && scale >= 1e-30f, SAS_ERR_INVALID_ARG, "scale must be finite and >= 1e-30");
  REQUIRE(aligned16(Q) && aligned16(K) && aligned16(V), SAS_ERR_INVALID_ARG, "Q, K, V must be 16-byte aligned");
  REQUIRE((long long)B * Hq * n * d < (1ll << 40), SAS_ERR_UNSUPPORTED, "tensor too large");
  // one (batch, head) slice of K / V is addressed by a 31-bit buffer resource
  REQUIRE((long long)n * d * 2 < (1ll << 31), SAS_ERR_UNSUPPORTED, "n * d * 2 bytes must be < 2^31");
  REQUIRE((long long)B * Hkv * (n / 64) < (1ll << 31) / 4, SAS_ERR_UNSUPPORTED, "too many blocks");
  REQUIRE((long long)(n / 64) * (kcap > 0 ? kcap : 1) < (1ll << 31), SAS_ERR_UNSUPPORTED, "n/64 * kcap too large");
  (void)logg;
  return SAS_OK;
}

}  // namespace

extern "C" {

const char* sas_version(void) { return "sas-mi355x 0.1.0 gfx950"; }

const char* sas_status_string(sas_status st) {
  switch (st) {
    case SAS_OK: return "SAS_OK";
    case SAS_ERR_INVALID_ARG: return "SAS_ERR_INVALID_ARG";
    case SAS_ERR_UNSUPPORTED: return "SAS_ERR_UNSUPPORTED";
    case SAS_ERR_WORKSPACE: return "SAS_ERR_WORKSPACE";
    case SAS_ERR_HIP: return "SAS_ERR_HIP";
  }
  return "SAS_ERR_UNKNOWN";
}

const char* sas_last_error(void) { return g_last_error.c_str(); }

sas_status sas_gates(const float* s, int B, int H, int rows, int cols, int ld, int mode,
                     const int32_t* row_valid, float* lse, float* g, void* stream) {
  sas_status st = check_rows(s, B, H, rows, cols, ld, mode, row_valid);
  if (st != SAS_OK) return st;
  REQUIRE(lse != nullptr, SAS_ERR_INVALID_ARG, "lse is NULL");
  sas::SelectArgs a{};
  a.s = s; a.R = (long long)B * H * rows; a.H = H; a.rows = rows; a.cols = cols; a.ld = ld;
  a.mode = mode; a.row_valid = row_valid; a.do_select = 0; a.lse = lse; a.g = g;
  return hip_result(sas::launch_select(a, (hipStream_t)stream), "sas_gates launch");
}

sas_status sas_gates_bwd(const float* s, int B, int H, int rows, int cols, int ld, int mode,
                         const int32_t* row_valid, int gate, const float* lse, const int32_t* idx,
                         const int32_t* cnt, const float* dg, int kcap, float* ds, void* stream) {
  sas_status st = check_rows(s, B, H, rows, cols, ld, mode, row_valid);
  if (st != SAS_OK) return st;
  REQUIRE(gate >= SAS_GATE_SOFTMAX && gate <= SAS_GATE_EXP, SAS_ERR_INVALID_ARG, "bad gate %d", gate);
  REQUIRE(cnt != nullptr && ds != nullptr, SAS_ERR_INVALID_ARG, "cnt and ds must be non-NULL");
  REQUIRE(lse != nullptr || gate == SAS_GATE_SIGMOID || gate == SAS_GATE_EXP, SAS_ERR_INVALID_ARG,
          "lse must be non-NULL for the softmax gates");
  REQUIRE(kcap >= 0 && kcap <= 8192, SAS_ERR_INVALID_ARG, "kcap=%d out of [0, 8192]", kcap);
  REQUIRE(kcap == 0 || (idx != nullptr && dg != nullptr), SAS_ERR_INVALID_ARG, "idx and dg must be non-NULL");
  REQUIRE((const void*)ds != (const void*)s, SAS_ERR_INVALID_ARG, "ds must not alias s");
  sas::GatesBwdArgs a{};
  a.s = s; a.R = (long long)B * H * rows; a.H = H; a.rows = rows; a.cols = cols; a.ld = ld;
  a.mode = mode; a.row_valid = row_valid; a.lse = lse; a.idx = idx; a.cnt = cnt; a.dg = dg;
  a.kcap = kcap; a.gate = gate; a.ds = ds;
  return hip_result(sas::launch_gates_bwd(a, (hipStream_t)stream), "sas_gates_bwd launch");
}

sas_status sas_topk_select(const float* s, int B, int H, int rows, int cols, int ld, int mode,
                           const int32_t* row_valid, int topk, int scope, int gate, int kcap,
                           int32_t* idx, int32_t* cnt, float* lse, float* logg, void* stream) {
  sas_status st = check_rows(s, B, H, rows, cols, ld, mode, row_valid);
  if (st != SAS_OK) return st;
  REQUIRE(scope == SAS_SCOPE_SPARSE || scope == SAS_SCOPE_FULL, SAS_ERR_INVALID_ARG, "bad scope %d", scope);
  REQUIRE(gate >= SAS_GATE_SOFTMAX && gate <= SAS_GATE_EXP, SAS_ERR_INVALID_ARG, "bad gate %d", gate);
  REQUIRE(topk >= 0, SAS_ERR_INVALID_ARG, "topk=%d < 0", topk);
  REQUIRE(cnt != nullptr, SAS_ERR_INVALID_ARG, "cnt is NULL");
  // most history blocks any row can have: rows - 1 in PREFILL (row j has j), cols in DECODE
  const int maxvalid = mode == SAS_ROWS_PREFILL ? (rows - 1 < cols ? rows - 1 : cols) : cols;
  const int need = scope == SAS_SCOPE_FULL ? maxvalid : (topk < maxvalid ? topk : maxvalid);
  REQUIRE(kcap >= need, SAS_ERR_INVALID_ARG, "kcap=%d < %d blocks a row may keep", kcap, need);
  REQUIRE(kcap == 0 || idx != nullptr, SAS_ERR_INVALID_ARG, "idx is NULL");
  sas::SelectArgs a{};
  a.s = s; a.R = (long long)B * H * rows; a.H = H; a.rows = rows; a.cols = cols; a.ld = ld;
  a.mode = mode; a.row_valid = row_valid; a.topk = topk; a.full = scope == SAS_SCOPE_FULL;
  a.kcap = kcap; a.do_select = 1; a.gate = gate; a.idx = idx; a.cnt = cnt; a.lse = lse; a.logg = logg;
  return hip_result(sas::launch_select(a, (hipStream_t)stream), "sas_topk_select launch");
}

sas_status sas_attn_fwd(const void* Q, const void* K, const void* V, const int32_t* idx,
                        const int32_t* cnt, const float* logg, int B, int Hq, int Hkv, int n,
                        int d, int block, int kcap, float scale, int placement, void* O,
                        float* lse_rows, void* stream) {
  sas_status st = check_attn(Q, K, V, idx, cnt, logg, B, Hq, Hkv, n, d, block, kcap, scale);
  if (st != SAS_OK) return st;
  REQUIRE(placement == SAS_GATE_INSIDE || placement == SAS_GATE_OUTSIDE, SAS_ERR_INVALID_ARG,
          "bad placement %d", placement);
  REQUIRE(O != nullptr && lse_rows != nullptr, SAS_ERR_INVALID_ARG, "O and lse_rows must be non-NULL");
  REQUIRE(aligned16(O), SAS_ERR_INVALID_ARG, "O must be 16-byte aligned");
  sas::AttnArgs a{};
  a.Q = (const uint16_t*)Q; a.K = (const uint16_t*)K; a.V = (const uint16_t*)V;
  a.idx = idx; a.cnt = cnt; a.logg = logg;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.n = n; a.d = d; a.kcap = kcap; a.scale = scale;
  a.gate_out = placement == SAS_GATE_OUTSIDE;
  a.Oout = (uint16_t*)O; a.lse_rows = lse_rows;
  return hip_result(sas::launch_fwd(a, (hipStream_t)stream), "sas_attn_fwd launch");
}

size_t sas_attn_bwd_workspace_size(int B, int Hq, int Hkv, int n, int d, int block, int kcap) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || n <= 0 || block != 64 || n % 64 != 0 || kcap < 0) return 0;
  if (Hq % Hkv != 0 || (d != 64 && d != 128)) return 0;
  return sas::bwd_workspace_bytes(B, Hq, Hkv, n, d, kcap);
}

sas_status sas_attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* lse_rows, const int32_t* idx,
                        const int32_t* cnt, const float* logg, int B, int Hq, int Hkv, int n,
                        int d, int block, int kcap, float scale, int placement, float* dQ,
                        float* dK, float* dV, float* dg, void* ws, size_t ws_bytes, void* stream) {
  sas_status st = check_attn(Q, K, V, idx, cnt, logg, B, Hq, Hkv, n, d, block, kcap, scale);
  if (st != SAS_OK) return st;
  REQUIRE(placement == SAS_GATE_INSIDE || placement == SAS_GATE_OUTSIDE, SAS_ERR_INVALID_ARG,
          "bad placement %d", placement);
  REQUIRE(O && dO && lse_rows, SAS_ERR_INVALID_ARG, "O, dO and lse_rows must be non-NULL");
  REQUIRE(dQ && dK && dV, SAS_ERR_INVALID_ARG, "dQ, dK and dV must be non-NULL");
  REQUIRE(kcap == 0 || dg != nullptr, SAS_ERR_INVALID_ARG, "dg is NULL");
  // the key-major pass addresses the rows of one KV group with 31-bit buffer offsets
  REQUIRE((long long)(Hq / Hkv) * n * d * 2 < (1ll << 31), SAS_ERR_UNSUPPORTED,
          "(Hq/Hkv) * n * d * 2 bytes must be < 2^31 for the backward pass");
  REQUIRE(aligned16(O) && aligned16(dO) && aligned16(dQ) && aligned16(dK) && aligned16(dV),
          SAS_ERR_INVALID_ARG, "O, dO, dQ, dK, dV must be 16-byte aligned");
  const size_t need = sas::bwd_workspace_bytes(B, Hq, Hkv, n, d, kcap);
  REQUIRE(ws != nullptr && ws_bytes >= need, SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), SAS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  sas::AttnArgs a{};
  a.Q = (const uint16_t*)Q; a.K = (const uint16_t*)K; a.V = (const uint16_t*)V;
  a.O = (const uint16_t*)O; a.dO = (const uint16_t*)dO;
  a.idx = idx; a.cnt = cnt; a.logg = logg;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.n = n; a.d = d; a.kcap = kcap; a.scale = scale;
  a.gate_out = placement == SAS_GATE_OUTSIDE;
  a.lse_rows = (float*)lse_rows; a.dQ = dQ; a.dK = dK; a.dV = dV; a.dg = dg;
  return hip_result(sas::launch_bwd(a, ws, (hipStream_t)stream), "sas_attn_bwd launch");
}

size_t sas_decode_workspace_size(int B, int Hq, int Hkv, int d, int kcap) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || kcap < 0 || Hq % Hkv != 0 || (d != 64 && d != 128)) return 0;
  return sas::decode_workspace_bytes(B, Hq, Hkv, d, kcap);
}

namespace {

sas_status check_decode(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len, int Lmax,
                        const int32_t* idx, const int32_t* cnt, int B, int Hq, int Hkv, int d, int block,
                        int kcap, float scale, const void* o) {
  REQUIRE(q && Kc && Vc && kv_len && cnt && o, SAS_ERR_INVALID_ARG, "q, Kc, Vc, kv_len, cnt, o must be non-NULL");
  REQUIRE(kcap == 0 || idx != nullptr, SAS_ERR_INVALID_ARG, "idx is NULL");
  REQUIRE(B > 0 && Hq > 0 && Hkv > 0 && Lmax > 0, SAS_ERR_INVALID_ARG, "B, Hq, Hkv, Lmax must be > 0");
  REQUIRE(Hq % Hkv == 0, SAS_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  const int G = Hq / Hkv;
  REQUIRE(G <= 32, SAS_ERR_UNSUPPORTED, "decode supports Hq/Hkv <= 32 (got %d)", G);
  REQUIRE((long long)Lmax * d * 2 < (1ll << 31), SAS_ERR_UNSUPPORTED,
          "Lmax * d * 2 bytes must be < 2^31 (one cache row range per buffer resource)");
  REQUIRE(block == 64, SAS_ERR_UNSUPPORTED, "block must be 64 (got %d)", block);
  REQUIRE(d == 64 || d == 128, SAS_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  REQUIRE(kcap >= 0 && kcap <= 8192, SAS_ERR_INVALID_ARG, "kcap=%d out of [0, 8192]", kcap);
  REQUIRE(isfinite(scale) && scale > 0.0f, SAS_ERR_INVALID_ARG, "scale must be finite and > 0");
  REQUIRE(aligned16(q) && aligned16(Kc) && aligned16(Vc) && aligned16(o), SAS_ERR_INVALID_ARG,
          "q, Kc, Vc, o must be 16-byte aligned");
  return SAS_OK;
}

sas::DecodeArgs decode_args(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len, int Lmax,
                            const int32_t* idx, const int32_t* cnt, const float* logg, int B, int Hq, int Hkv,
                            int d, int kcap, float scale, void* o) {
  sas::DecodeArgs a{};
  a.q = (const uint16_t*)q; a.Kc = (const uint16_t*)Kc; a.Vc = (const uint16_t*)Vc;
  a.kv_len = kv_len; a.Lmax = Lmax; a.idx = idx; a.cnt = cnt; a.logg = logg;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.kcap = kcap; a.scale = scale;
  a.o = (uint16_t*)o;
  return a;
}

// Scratch of sas_decode_noalloc: the partial softmax states of block lists split over
// several workgroups. Each device the library runs on holds its own copy until the process
// ends; in host code `scratch` only names the symbol, its device address comes from
// hipGetSymbolAddress, looked up once per device and kept.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
__device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sas_status decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SAS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  REQUIRE(dev >= 0 && dev < kMaxDevices, SAS_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev,
          kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(SAS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SAS_OK;
}

}  // namespace

sas_status sas_decode(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                      int Lmax, const int32_t* idx, const int32_t* cnt, const float* logg,
                      int B, int Hq, int Hkv, int d, int block, int kcap, float scale, void* o,
                      void* ws, size_t ws_bytes, void* stream) {
  const sas_status chk = check_decode(q, Kc, Vc, kv_len, Lmax, idx, cnt, B, Hq, Hkv, d, block, kcap, scale, o);
  if (chk != SAS_OK) return chk;
  const size_t need = sas::decode_workspace_bytes(B, Hq, Hkv, d, kcap);
  REQUIRE(ws != nullptr && ws_bytes >= need, SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), SAS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  sas::DecodeArgs a = decode_args(q, Kc, Vc, kv_len, Lmax, idx, cnt, logg, B, Hq, Hkv, d, kcap, scale, o);
  a.part = (float*)ws;
  return hip_result(sas::launch_decode(a, (hipStream_t)stream), "sas_decode launch");
}

sas_status sas_decode_topk(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                           int Lmax, const float* s, int ld, int topk, int B, int Hq, int Hkv,
                           int d, int block, float scale, void* o, int32_t* idx, int32_t* cnt,
                           void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(s != nullptr, SAS_ERR_INVALID_ARG, "s must be non-NULL");
  REQUIRE((idx == nullptr) == (cnt == nullptr), SAS_ERR_INVALID_ARG, "idx and cnt must both be given or both NULL");
  REQUIRE(topk >= 1, SAS_ERR_INVALID_ARG, "topk=%d must be >= 1", topk);
  REQUIRE(topk <= sas::kDecSelMax, SAS_ERR_UNSUPPORTED, "topk=%d above %d: use sas_topk_select and sas_decode", topk,
          sas::kDecSelMax);
  REQUIRE(Lmax > 0 && (Lmax - 1) / 64 <= sas::kDecSelMaxCols, SAS_ERR_UNSUPPORTED,
          "Lmax=%d: more than %d history blocks per row; use sas_topk_select and sas_decode", Lmax,
          sas::kDecSelMaxCols);
  REQUIRE(ld >= (Lmax - 1) / 64, SAS_ERR_INVALID_ARG, "ld=%d below the %d history blocks of Lmax=%d", ld,
          (Lmax - 1) / 64, Lmax);
  // cnt is an output here: check_decode's input checks are met with a stand-in pointer
  const int32_t dummy = 0;
  const sas_status chk = check_decode(q, Kc, Vc, kv_len, Lmax, &dummy, &dummy, B, Hq, Hkv, d, block, topk, scale, o);
  if (chk != SAS_OK) return chk;
  const size_t need = sas::decode_workspace_bytes(B, Hq, Hkv, d, topk);
  REQUIRE(ws != nullptr && ws_bytes >= need, SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), SAS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  sas::DecodeArgs a = decode_args(q, Kc, Vc, kv_len, Lmax, nullptr, nullptr, nullptr, B, Hq, Hkv, d, topk, scale, o);
  a.part = (float*)ws;
  a.s = s;
  a.s_ld = ld;
  a.topk = topk;
  a.idx_out = idx;
  a.cnt_out = cnt;
  return hip_result(sas::launch_decode(a, (hipStream_t)stream), "sas_decode_topk launch");
}

sas_status sas_decode_noalloc(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                              int Lmax, const int32_t* idx, const int32_t* cnt, const float* logg,
                              int B, int Hq, int Hkv, int d, int block, int kcap, float scale, void* o,
                              void* stream) {
  const sas_status chk = check_decode(q, Kc, Vc, kv_len, Lmax, idx, cnt, B, Hq, Hkv, d, block, kcap, scale, o);
  if (chk != SAS_OK) return chk;
  sas::DecodeArgs a = decode_args(q, Kc, Vc, kv_len, Lmax, idx, cnt, logg, B, Hq, Hkv, d, kcap, scale, o);
  sas::decode_plan(a);
  const size_t need = sas::decode_part_bytes(a);
  REQUIRE(need <= kDecodeScratchBytes, SAS_ERR_UNSUPPORTED,
          "these sizes need %zu bytes of partial states, beyond the %zu-byte device scratch of sas_decode_noalloc",
          need, kDecodeScratchBytes);
  void* ptr = nullptr;
  const sas_status sst = decode_scratch(&ptr);
  if (sst != SAS_OK) return sst;
  a.part = (float*)ptr;
  return hip_result(sas::launch_decode(a, (hipStream_t)stream), "sas_decode_noalloc launch");
}

sas_status sas_decode_early_stop(const void* q, const void* Kc, const void* Vc, const int32_t* kv_len,
                                 int Lmax, const int32_t* idx, const int32_t* cnt, const float* order,
                                 int B, int Hq, int Hkv, int d, int block, int kcap, float scale,
                                 float tau, void* o, int32_t* used, void* stream) {
  REQUIRE(q && Kc && Vc && kv_len && cnt && order && o, SAS_ERR_INVALID_ARG,
          "q, Kc, Vc, kv_len, cnt, order, o must be non-NULL");
  REQUIRE(kcap == 0 || idx != nullptr, SAS_ERR_INVALID_ARG, "idx is NULL");
  REQUIRE(B > 0 && Hq > 0 && Hkv > 0 && Lmax > 0, SAS_ERR_INVALID_ARG, "B, Hq, Hkv, Lmax must be > 0");
  REQUIRE(Hq % Hkv == 0, SAS_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  REQUIRE(Hq / Hkv <= 32, SAS_ERR_UNSUPPORTED, "decode supports Hq/Hkv <= 32 (got %d)", Hq / Hkv);
  REQUIRE((long long)Lmax * d * 2 < (1ll << 31), SAS_ERR_UNSUPPORTED,
          "Lmax * d * 2 bytes must be < 2^31 (one cache row range per buffer resource)");
  REQUIRE(block == 64, SAS_ERR_UNSUPPORTED, "block must be 64 (got %d)", block);
  REQUIRE(d == 64 || d == 128, SAS_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  REQUIRE(kcap >= 0 && kcap <= 63, SAS_ERR_UNSUPPORTED, "the early stop sorts at most 63 blocks (kcap=%d)", kcap);
  REQUIRE(isfinite(scale) && scale > 0.0f, SAS_ERR_INVALID_ARG, "scale must be finite and > 0");
  REQUIRE(isfinite(tau) && tau >= 0.0f, SAS_ERR_INVALID_ARG, "tau must be finite and >= 0");
  REQUIRE(aligned16(q) && aligned16(Kc) && aligned16(Vc) && aligned16(o), SAS_ERR_INVALID_ARG,
          "q, Kc, Vc, o must be 16-byte aligned");
  sas::DecodeArgs a{};
  a.q = (const uint16_t*)q; a.Kc = (const uint16_t*)Kc; a.Vc = (const uint16_t*)Vc;
  a.kv_len = kv_len; a.Lmax = Lmax; a.idx = idx; a.cnt = cnt; a.logg = nullptr;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.kcap = kcap; a.scale = scale;
  a.o = (uint16_t*)o; a.part = nullptr;
  a.order = order; a.tau = tau; a.used = used;
  return hip_result(sas::launch_decode(a, (hipStream_t)stream), "sas_decode_early_stop launch");
}

static sas_status check_decode_paged(const void* q, const void* Kpool, const void* Vpool, int num_pages,
                                     const int32_t* page_table, int max_pages, const int32_t* kv_len,
                                     const int32_t* idx, const int32_t* cnt, int B, int Hq, int Hkv, int d,
                                     int block, int kcap, float scale, const void* o) {
  REQUIRE(q && Kpool && Vpool && page_table && kv_len && cnt && o, SAS_ERR_INVALID_ARG,
          "q, Kpool, Vpool, page_table, kv_len, cnt, o must be non-NULL");
  REQUIRE(kcap == 0 || idx != nullptr, SAS_ERR_INVALID_ARG, "idx is NULL");
  REQUIRE(B > 0 && Hq > 0 && Hkv > 0 && num_pages > 0 && max_pages > 0, SAS_ERR_INVALID_ARG,
          "B, Hq, Hkv, num_pages, max_pages must be > 0");
  REQUIRE(Hq % Hkv == 0, SAS_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  REQUIRE(Hq / Hkv <= 32, SAS_ERR_UNSUPPORTED, "decode supports Hq/Hkv <= 32 (got %d)", Hq / Hkv);
  REQUIRE(block == 64, SAS_ERR_UNSUPPORTED, "block (page size) must be 64 (got %d)", block);
  REQUIRE(d == 64 || d == 128, SAS_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  REQUIRE((long long)max_pages * 64 < (1ll << 31), SAS_ERR_UNSUPPORTED, "max_pages too large");
  REQUIRE(kcap >= 0 && kcap <= 8192, SAS_ERR_INVALID_ARG, "kcap=%d out of [0, 8192]", kcap);
  REQUIRE(isfinite(scale) && scale > 0.0f, SAS_ERR_INVALID_ARG, "scale must be finite and > 0");
  REQUIRE(aligned16(q) && aligned16(Kpool) && aligned16(Vpool) && aligned16(o), SAS_ERR_INVALID_ARG,
          "q, Kpool, Vpool, o must be 16-byte aligned");
  return SAS_OK;
}

static sas::DecodeArgs decode_paged_args(const void* q, const void* Kpool, const void* Vpool, int num_pages,
                                         const int32_t* page_table, int max_pages, const int32_t* kv_len,
                                         const int32_t* idx, const int32_t* cnt, const float* logg, int B,
                                         int Hq, int Hkv, int d, int kcap, float scale, void* o, void* ws) {
  sas::DecodeArgs a{};
  a.q = (const uint16_t*)q; a.Kc = (const uint16_t*)Kpool; a.Vc = (const uint16_t*)Vpool;
  a.kv_len = kv_len; a.Lmax = (long long)max_pages * 64; a.idx = idx; a.cnt = cnt; a.logg = logg;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.d = d; a.kcap = kcap; a.scale = scale;
  a.o = (uint16_t*)o; a.part = (float*)ws;
  a.page_table = page_table; a.max_pages = max_pages; a.num_pages = num_pages;
  return a;
}

sas_status sas_decode_paged(const void* q, const void* Kpool, const void* Vpool, int num_pages,
                            const int32_t* page_table, int max_pages, const int32_t* kv_len,
                            const int32_t* idx, const int32_t* cnt, const float* logg, int B, int Hq,
                            int Hkv, int d, int block, int kcap, float scale, void* o, void* ws,
                            size_t ws_bytes, void* stream) {
  const sas_status chk = check_decode_paged(q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, idx, cnt, B,
                                            Hq, Hkv, d, block, kcap, scale, o);
  if (chk != SAS_OK) return chk;
  const size_t need = sas::decode_workspace_bytes(B, Hq, Hkv, d, kcap);
  REQUIRE(ws != nullptr && ws_bytes >= need, SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), SAS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const sas::DecodeArgs a = decode_paged_args(q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, idx, cnt,
                                              logg, B, Hq, Hkv, d, kcap, scale, o, ws);
  return hip_result(sas::launch_decode(a, (hipStream_t)stream), "sas_decode_paged launch");
}

sas_status sas_decode_paged_topk(const void* q, const void* Kpool, const void* Vpool, int num_pages,
                                 const int32_t* page_table, int max_pages, const int32_t* kv_len,
                                 const float* s, int ld, int topk, int B, int Hq, int Hkv, int d,
                                 int block, float scale, void* o, int32_t* idx, int32_t* cnt, void* ws,
                                 size_t ws_bytes, void* stream) {
  REQUIRE(s != nullptr, SAS_ERR_INVALID_ARG, "s must be non-NULL");
  REQUIRE((idx == nullptr) == (cnt == nullptr), SAS_ERR_INVALID_ARG, "idx and cnt must both be given or both NULL");
  REQUIRE(topk >= 1, SAS_ERR_INVALID_ARG, "topk=%d must be >= 1", topk);
  REQUIRE(topk <= sas::kDecSelMax, SAS_ERR_UNSUPPORTED, "topk=%d above %d: use sas_topk_select and sas_decode_paged",
          topk, sas::kDecSelMax);
  REQUIRE(max_pages > 0 && max_pages - 1 <= sas::kDecSelMaxCols, SAS_ERR_UNSUPPORTED,
          "max_pages=%d: more than %d history blocks per row; use sas_topk_select and sas_decode_paged", max_pages,
          sas::kDecSelMaxCols);
  REQUIRE(ld >= max_pages - 1, SAS_ERR_INVALID_ARG, "ld=%d below the %d history blocks of max_pages=%d", ld,
          max_pages - 1, max_pages);
  // cnt is an output here: the input checks are met with a stand-in pointer
  const int32_t dummy = 0;
  const sas_status chk = check_decode_paged(q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, &dummy,
                                            &dummy, B, Hq, Hkv, d, block, topk, scale, o);
  if (chk != SAS_OK) return chk;
  const size_t need = sas::decode_workspace_bytes(B, Hq, Hkv, d, topk);
  REQUIRE(ws != nullptr && ws_bytes >= need, SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), SAS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  sas::DecodeArgs a = decode_paged_args(q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, nullptr, nullptr,
                                        nullptr, B, Hq, Hkv, d, topk, scale, o, ws);
  a.s = s;
  a.s_ld = ld;
  a.topk = topk;
  a.idx_out = idx;
  a.cnt_out = cnt;
  return hip_result(sas::launch_decode(a, (hipStream_t)stream), "sas_decode_paged_topk launch");
}

sas_status sas_pool_keys(const void* Kc, int B, int Hkv, int Lmax, int d, const int32_t* kv_len,
                         int first_block, void* kbar, void* stream) {
  REQUIRE(Kc && kv_len && kbar, SAS_ERR_INVALID_ARG, "Kc, kv_len and kbar must be non-NULL");
  REQUIRE(B > 0 && Hkv > 0 && Lmax > 0, SAS_ERR_INVALID_ARG, "B, Hkv, Lmax must be > 0");
  REQUIRE(Lmax % 64 == 0, SAS_ERR_INVALID_ARG, "Lmax=%d is not a multiple of 64", Lmax);
  REQUIRE(d == 64 || d == 128, SAS_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  const int C = Lmax / 64;
  REQUIRE(first_block >= 0 && first_block <= C, SAS_ERR_INVALID_ARG, "first_block=%d out of [0, %d]", first_block, C);
  REQUIRE((long long)B * Hkv * (C - first_block) < (1ll << 31), SAS_ERR_UNSUPPORTED, "too many blocks");
  REQUIRE(aligned16(Kc) && aligned16(kbar), SAS_ERR_INVALID_ARG, "Kc and kbar must be 16-byte aligned");
  sas::PoolArgs a{};
  a.K = (const uint16_t*)Kc; a.B = B; a.Hkv = Hkv; a.Lmax = Lmax; a.C = C; a.d = d;
  a.kv_len = kv_len; a.first_block = first_block; a.nblk = C - first_block; a.kbar = (uint16_t*)kbar;
  return hip_result(sas::launch_pool(a, (hipStream_t)stream), "sas_pool_keys launch");
}

sas_status sas_decode_select(const void* q, const void* kbar, int B, int Hq, int Hkv, int d, int C,
                             const int32_t* kv_len, float scale, int topk, int kcap, float* s,
                             int32_t* idx, int32_t* cnt, float* lse, float* logg, void* stream) {
  REQUIRE(q && kbar && kv_len && s && cnt, SAS_ERR_INVALID_ARG, "q, kbar, kv_len, s, cnt must be non-NULL");
  REQUIRE(kcap == 0 || idx != nullptr, SAS_ERR_INVALID_ARG, "idx is NULL");
  REQUIRE(B > 0 && Hq > 0 && Hkv > 0 && C > 0, SAS_ERR_INVALID_ARG, "B, Hq, Hkv, C must be > 0");
  REQUIRE(Hq % Hkv == 0, SAS_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  REQUIRE(d == 64 || d == 128, SAS_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  REQUIRE(C <= 8192, SAS_ERR_UNSUPPORTED, "C=%d exceeds 8192 blocks", C);
  REQUIRE(topk >= 0, SAS_ERR_INVALID_ARG, "topk must be >= 0");
  REQUIRE(kcap >= std::min(topk, C) && kcap <= 8192, SAS_ERR_INVALID_ARG,
          "kcap=%d must be in [min(topk, C), 8192]", kcap);
  REQUIRE(isfinite(scale) && scale > 0.0f, SAS_ERR_INVALID_ARG, "scale must be finite and > 0");
  REQUIRE(aligned16(q) && aligned16(kbar), SAS_ERR_INVALID_ARG, "q and kbar must be 16-byte aligned");
  REQUIRE((long long)B * Hkv * C * d * 2 < (1ll << 40), SAS_ERR_UNSUPPORTED, "pooled cache too large");
  sas::DecSelArgs a{};
  a.q = (const uint16_t*)q; a.kbar = (const uint16_t*)kbar; a.B = B; a.Hq = Hq; a.Hkv = Hkv;
  a.G = Hq / Hkv; a.d = d; a.C = C; a.kv_len = kv_len; a.scale = scale; a.topk = topk; a.kcap = kcap;
  a.s = s; a.idx = idx; a.cnt = cnt; a.lse = lse; a.logg = logg;
  return hip_result(sas::launch_decode_select(a, (hipStream_t)stream), "sas_decode_select launch");
}

// Workspace of sas_decode_long: the decode's partial states, then the candidate slots
// (scores, then blocks), each part 256-byte aligned. 0 on invalid sizes.
static size_t decode_long_layout(int B, int Hq, int Hkv, int d, int C, int topk, int* cch, int* cld,
                                 size_t* cand_off) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || (d != 64 && d != 128) || C <= 0 || C > 8192 || topk < 1 ||
      topk > sas::kDecSelMax)
    return 0;
  const int ch = sas::decode_cand_chunk(C, topk, d);
  if (ch == 0) return 0;
  const int ld = (C + ch - 1) / ch * topk;
  const size_t part = (sas::decode_workspace_bytes(B, Hq, Hkv, d, topk) + 255) / 256 * 256;
  const size_t slots = (size_t)B * Hkv * ld;
  if (cch) *cch = ch;
  if (cld) *cld = ld;
  if (cand_off) *cand_off = part;
  return part + (slots * 4 + 255) / 256 * 256 + slots * 4;
}

size_t sas_decode_long_workspace_size(int B, int Hq, int Hkv, int d, int C, int topk) {
  return decode_long_layout(B, Hq, Hkv, d, C, topk, nullptr, nullptr, nullptr);
}

// The two launches of a long-context decode step (candidates, then the decode ranking them)
// for a decode already described by `a` (caches, paging, sizes, scale, o): checks of kbar,
// topk, C and the workspace, then the launches.
static sas_status decode_long_launch(sas::DecodeArgs a, const void* kbar, int C, int topk, int32_t* idx,
                                     int32_t* cnt, void* ws, size_t ws_bytes, void* stream, const char* what) {
  int cch = 0, cld = 0;
  size_t cand_off = 0;
  const size_t need = decode_long_layout(a.B, a.Hq, a.Hkv, a.d, C, topk, &cch, &cld, &cand_off);
  REQUIRE(need > 0, SAS_ERR_UNSUPPORTED, "no candidate layout for C=%d, topk=%d", C, topk);
  REQUIRE(ws != nullptr && ws_bytes >= need, SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  REQUIRE(aligned16(ws), SAS_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  const size_t slots = (size_t)a.B * a.Hkv * cld;
  float* cs = (float*)((char*)ws + cand_off);
  int32_t* ci = (int32_t*)((char*)ws + cand_off + (slots * 4 + 255) / 256 * 256);

  sas::DecSelArgs sa{};
  sa.q = a.q; sa.kbar = (const uint16_t*)kbar; sa.B = a.B; sa.Hq = a.Hq; sa.Hkv = a.Hkv;
  sa.G = a.Hq / a.Hkv; sa.d = a.d; sa.C = C; sa.kv_len = a.kv_len; sa.scale = a.scale; sa.topk = topk;
  sa.cs = cs; sa.ci = ci; sa.cch = cch; sa.cld = cld;
  sa.hist_cap = (int)((a.Lmax - 1) / 64);   // kv_len past the cache is clamped, as in the decode
  const sas_status st = hip_result(sas::launch_decode_candidates(sa, (hipStream_t)stream), what);
  if (st != SAS_OK) return st;
  a.part = (float*)ws;
  a.s = cs;
  a.s_ld = cld;
  a.s_id = ci;
  a.topk = topk;
  a.idx_out = idx;
  a.cnt_out = cnt;
  return hip_result(sas::launch_decode(a, (hipStream_t)stream), what);
}

static sas_status check_decode_long(const void* kbar, int C, int topk, int hist_max, const int32_t* idx,
                                    const int32_t* cnt) {
  REQUIRE(kbar != nullptr, SAS_ERR_INVALID_ARG, "kbar must be non-NULL");
  REQUIRE((idx == nullptr) == (cnt == nullptr), SAS_ERR_INVALID_ARG, "idx and cnt must both be given or both NULL");
  REQUIRE(topk >= 1, SAS_ERR_INVALID_ARG, "topk=%d must be >= 1", topk);
  REQUIRE(topk <= sas::kDecSelMax, SAS_ERR_UNSUPPORTED,
          "topk=%d above %d: use sas_decode_select and sas_decode", topk, sas::kDecSelMax);
  REQUIRE(C >= 1 && C <= 8192, SAS_ERR_UNSUPPORTED, "C=%d out of [1, 8192] pooled blocks", C);
  REQUIRE(hist_max <= C, SAS_ERR_INVALID_ARG, "C=%d pooled blocks cannot hold %d history blocks", C, hist_max);
  REQUIRE(aligned16(kbar), SAS_ERR_INVALID_ARG, "kbar must be 16-byte aligned");
  return SAS_OK;
}

sas_status sas_decode_long(const void* q, const void* kbar, int C, const void* Kc, const void* Vc,
                           const int32_t* kv_len, int Lmax, int topk, int B, int Hq, int Hkv, int d,
                           int block, float scale, void* o, int32_t* idx, int32_t* cnt, void* ws,
                           size_t ws_bytes, void* stream) {
  REQUIRE(Lmax > 0, SAS_ERR_INVALID_ARG, "Lmax must be > 0");
  const sas_status lc = check_decode_long(kbar, C, topk, (Lmax - 1) / 64, idx, cnt);
  if (lc != SAS_OK) return lc;
  // cnt is an output here: check_decode's input checks are met with a stand-in pointer
  const int32_t dummy = 0;
  const sas_status chk = check_decode(q, Kc, Vc, kv_len, Lmax, &dummy, &dummy, B, Hq, Hkv, d, block, topk, scale, o);
  if (chk != SAS_OK) return chk;
  const sas::DecodeArgs a = decode_args(q, Kc, Vc, kv_len, Lmax, nullptr, nullptr, nullptr, B, Hq, Hkv, d, topk,
                                        scale, o);
  return decode_long_launch(a, kbar, C, topk, idx, cnt, ws, ws_bytes, stream, "sas_decode_long launch");
}

sas_status sas_decode_long_paged(const void* q, const void* kbar, const void* Kpool, const void* Vpool,
                                 int num_pages, const int32_t* page_table, int max_pages,
                                 const int32_t* kv_len, int topk, int B, int Hq, int Hkv, int d, int block,
                                 float scale, void* o, int32_t* idx, int32_t* cnt, void* ws, size_t ws_bytes,
                                 void* stream) {
  const sas_status lc = check_decode_long(kbar, max_pages, topk, max_pages - 1, idx, cnt);
  if (lc != SAS_OK) return lc;
  const int32_t dummy = 0;
  const sas_status chk = check_decode_paged(q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, &dummy,
                                            &dummy, B, Hq, Hkv, d, block, topk, scale, o);
  if (chk != SAS_OK) return chk;
  const sas::DecodeArgs a = decode_paged_args(q, Kpool, Vpool, num_pages, page_table, max_pages, kv_len, nullptr,
                                              nullptr, nullptr, B, Hq, Hkv, d, topk, scale, o, nullptr);
  return decode_long_launch(a, kbar, max_pages, topk, idx, cnt, ws, ws_bytes, stream,
                            "sas_decode_long_paged launch");
}

sas_status sas_pool_keys_paged(const void* Kpool, int num_pages, const int32_t* page_table, int max_pages,
                               int B, int Hkv, int d, const int32_t* kv_len, int first_block, void* kbar,
                               void* stream) {
  REQUIRE(Kpool && page_table && kv_len && kbar, SAS_ERR_INVALID_ARG,
          "Kpool, page_table, kv_len and kbar must be non-NULL");
  REQUIRE(B > 0 && Hkv > 0 && num_pages > 0 && max_pages > 0, SAS_ERR_INVALID_ARG,
          "B, Hkv, num_pages, max_pages must be > 0");
  REQUIRE(d == 64 || d == 128, SAS_ERR_UNSUPPORTED, "d must be 64 or 128 (got %d)", d);
  REQUIRE(max_pages <= 8192, SAS_ERR_UNSUPPORTED, "max_pages=%d above 8192", max_pages);
  REQUIRE(first_block >= 0 && first_block <= max_pages, SAS_ERR_INVALID_ARG, "first_block=%d out of [0, %d]",
          first_block, max_pages);
  REQUIRE(aligned16(Kpool) && aligned16(kbar), SAS_ERR_INVALID_ARG, "Kpool and kbar must be 16-byte aligned");
  sas::PoolArgs a{};
  a.K = (const uint16_t*)Kpool; a.B = B; a.Hkv = Hkv; a.Lmax = max_pages * 64; a.C = max_pages; a.d = d;
  a.kv_len = kv_len; a.first_block = first_block; a.nblk = max_pages - first_block; a.kbar = (uint16_t*)kbar;
  a.page_table = page_table; a.num_pages = num_pages;
  return hip_result(sas::launch_pool(a, (hipStream_t)stream), "sas_pool_keys_paged launch");
}

}  // extern "C"
