// Gate normalisation and Top-K block selection, one wavefront per score row.
//
// [SAS-ko] "무엇과 다른가", choice 2: g = softmax(s) over the row's valid history blocks,
// log g_m = s_m - LSE(s). [SAS-ja] "前提" / "仕組み" (Algorithm 2): the K best-scoring
// history blocks are attended. Selection compares the fp32 scores themselves; ties go to
// the lower block index, -0 equals +0 and NaN ranks as -inf.
//
// Each lane holds PL scores (element m = lane + 64 i, so loads are coalesced). The K-th
// largest order-preserving key is found by fixing its 32 bits from the top: a candidate
// bit stays set when at least K keys are >= the candidate, counted with one ballot per
// register. Blocks strictly above the threshold are kept; among the blocks equal to it the
// lowest indices fill the remaining places. A ballot prefix count writes the kept indices
// in ascending order without any sort.
#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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

template <int PL>
__global__ __launch_bounds__(256) void select_kernel(const SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.R) return;  // uniform per wave
  int valid;
  if (a.mode == 0) {
    valid = (int)(row % a.rows);
  } else {
    const long long b = row / ((long long)a.H * a.rows);
    valid = a.row_valid[b];
  }
  valid = min(max(valid, 0), a.cols);
  const float* srow = a.s + row * a.ld;

  float x[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int m = lane + 64 * i;
    float v = -INFINITY;
    if (m < valid) {
      v = srow[m];
      if (v != v) v = -INFINITY;  // NaN ranks as -inf
      if (v == 0.0f) v = 0.0f;    // -0 -> +0
    }
    x[i] = v;
  }

  // LSE over the valid scores.
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PL; ++i) mx = fmaxf(mx, x[i]);
  mx = wave_max(mx);
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < PL; ++i) sum += expf(x[i] - mx);
    sum = wave_sum(sum);
    lse = mx + logf(sum);
  }
  if (a.lse != nullptr && lane == 0 && (!a.do_select || a.gate == kGateSoftmax)) a.lse[row] = lse;
  if (a.g != nullptr) {
    float* grow = a.g + row * a.ld;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int m = lane + 64 * i;
      if (m < a.cols) grow[m] = (m < valid && lse != -INFINITY) ? expf(x[i] - lse) : 0.0f;
    }
  }
  if (!a.do_select) return;

  const int k = a.full ? valid : min(a.topk, valid);
  int32_t* idx_row = a.idx + row * a.kcap;
  float* lg_row = a.logg != nullptr ? a.logg + row * a.kcap : nullptr;
  if (k > 0) {
    uint32_t key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) key[i] = (lane + 64 * i < valid) ? order_key(x[i]) : 0u;
    // Valid keys are >= order_key(-inf) = 0x007FFFFF > 0, so padding (key 0) never reaches
    // the threshold.
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      int c = 0;
#pragma unroll
      for (int i = 0; i < PL; ++i) c += __popcll(__ballot(key[i] >= cand));
      if (c >= k) T = cand;
    }
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) n_gt += __popcll(__ballot(key[i] > T));
    const int need_eq = k - n_gt;
    const unsigned long long lt = (1ull << lane) - 1ull;
    // calls f(i, pos) for every kept register i of this lane, pos = its output slot
    auto walk = [&](auto&& f) {
      int base = 0, eq_before = 0;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const bool eq = key[i] == T;
        const unsigned long long beq = __ballot(eq);
        const int eq_rank = eq_before + __popcll(beq & lt);
        const bool sel = key[i] > T || (eq && eq_rank < need_eq);
        const unsigned long long bsel = __ballot(sel);
        if (sel) f(i, base + __popcll(bsel & lt));
        base += __popcll(bsel);
        eq_before += __popcll(beq);
      }
    };
    float norm = lse;   // the gate's normaliser (reported as lse)
    if (a.gate == kGateSoftmaxSelected) {
      float m = -INFINITY, sum = 0.0f;   // online LSE over the kept scores
      walk([&](int i, int) {
        if (x[i] > m) { sum = sum * expf(m - x[i]) + 1.0f; m = x[i]; }
        else if (x[i] != -INFINITY) sum += expf(x[i] - m);
      });
      const float wm = wave_max(m);
      sum = wave_sum(m == -INFINITY ? 0.0f : sum * expf(m - wm));
      norm = wm == -INFINITY ? -INFINITY : wm + logf(sum);
    } else if (a.gate != kGateSoftmax) {
      norm = 0.0f;
    }
    if (a.lse != nullptr && lane == 0 && a.gate != kGateSoftmax) a.lse[row] = norm;
    walk([&](int i, int pos) {
      idx_row[pos] = lane + 64 * i;
      if (lg_row != nullptr) lg_row[pos] = log_gate(a.gate, x[i], norm);
    });
  } else if (a.lse != nullptr && lane == 0 && a.gate != kGateSoftmax) {
    a.lse[row] = a.gate == kGateSoftmaxSelected ? -INFINITY : 0.0f;
  }
  for (int p = k + lane; p < a.kcap; p += 64) {
    idx_row[p] = -1;
    if (lg_row != nullptr) lg_row[p] = 0.0f;
  }
  if (lane == 0) a.cnt[row] = k;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.R + 3) / 4)), block(256);
  const int c = a.cols;
  ProfScope prof("select", st);
  if (c <= 64) hipLaunchKernelGGL(select_kernel<1>, grid, block, 0, st, a);
  else if (c <= 128) hipLaunchKernelGGL(select_kernel<2>, grid, block, 0, st, a);
  else if (c <= 256) hipLaunchKernelGGL(select_kernel<4>, grid, block, 0, st, a);
  else if (c <= 512) hipLaunchKernelGGL(select_kernel<8>, grid, block, 0, st, a);
  else if (c <= 1024) hipLaunchKernelGGL(select_kernel<16>, grid, block, 0, st, a);
  else if (c <= 2048) hipLaunchKernelGGL(select_kernel<32>, grid, block, 0, st, a);
  else if (c <= 4096) hipLaunchKernelGGL(select_kernel<64>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(select_kernel<128>, grid, block, 0, st, a);
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
    return expf(v - lse);
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
  c = wave_sum(c);
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
