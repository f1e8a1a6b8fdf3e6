// Long-context decode selection: block-mean key cache, block scores and Top-K.
//
// The SAS pages leave the selector network undefined; block importance is taken as the
// mean attention score over a block ([PBS-ja] "Sparser Block-Sparse Attention via Token
// Permutation", sections "3." (proxy scoring) and "4. 実装" (block selection by mean
// pooling)), averaged over the G query heads of a KV group because one score row serves
// the whole group. By linearity that mean equals scale * qbar . kbar_m, with qbar the mean
// of the group's queries and kbar_m the mean of block m's keys, so a decode step reads one
// pooled key (d bf16) per history block instead of its 64 keys. Selection then keeps the
// K best of those scores exactly as sas_topk_select does ([SAS-ja] "仕組み", Algorithm 2;
// ties to the lower block index, NaN as -inf), in one workgroup per row so that rows of up
// to 8192 blocks (512K tokens) finish in a few microseconds.
#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

namespace {

__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) x = -INFINITY;   // NaN ranks as -inf
  if (x == 0.0f) x = 0.0f;     // -0 equals +0
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ key pooling

// One workgroup per (sequence, KV head, block): thread t sums rows t / (D/8) + 256/(D/8) r
// of its 8-element column slice, LDS combines the row groups.
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const PoolArgs a) {
  constexpr int LPR = D / 8;          // threads per key row
  constexpr int RG = 256 / LPR;       // row groups
  __shared__ float part[RG][D];
  const long long wg = blockIdx.x;
  const int m = (int)(wg % a.nblk) + a.first_block;
  const long long bh = wg / a.nblk;
  const int b = (int)(bh / a.Hkv);
  if ((m + 1) * kBlock > a.kv_len[b] || m >= a.C) return;   // uniform per workgroup
  const int t = threadIdx.x, c = t % LPR, rg = t / LPR;
  const uint16_t* src = a.K + ((size_t)bh * a.Lmax + (size_t)m * kBlock) * D + 8 * c;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int r = rg; r < kBlock; r += RG) {
    const u16x8 v = ld16(src + (size_t)r * D);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += bf2f(v[i]);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[rg][8 * c + i] = acc[i];
  __syncthreads();
  if (t < D) {
    float sum = 0.0f;
#pragma unroll
    for (int g = 0; g < RG; ++g) sum += part[g][t];
    a.kbar[((size_t)bh * a.C + m) * D + t] = f2bf(sum * (1.0f / kBlock));
  }
}

// ------------------------------------------------------------------ Top-K per row

constexpr int kSelThreads = 256;
constexpr int kSelPer = kMaxCols / kSelThreads;   // 32 scores per thread, contiguous

// exclusive prefix sum over the workgroup and its total (all threads call it)
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelThreads / 64; ++i) {
    base += i < w ? wsum[i] : 0;
    tot += wsum[i];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kSelThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

// Top-K of one row by one workgroup. The K-th largest order key is found digit by digit
// (3 passes of 12, 10 and 10 bits, an LDS histogram per pass restricted to the keys that
// match the digits fixed so far); keys above it are kept and the remaining places go to
// the lowest-index keys equal to it. Thread t owns blocks 32 t .. 32 t + 31, so one prefix
// sum over the threads gives every kept block its output position in ascending order.
struct TopkSmem {
  int hist[4096];
  int wsum[kSelThreads / 64];
  float red[kSelThreads / 64];
  int pick[2];
};

__device__ __forceinline__ void topk_row(const DecSelArgs& a, long long row, TopkSmem& sm) {
  int* hist = sm.hist;
  int* wsum = sm.wsum;
  float* red = sm.red;
  int* pick = sm.pick;
  const int b = (int)(row / a.Hkv);
  const int n = min(max((a.kv_len[b] - 1) / kBlock, 0), a.C);
  const int k = min(a.topk, n);
  const int t = threadIdx.x;
  const int m0 = t * kSelPer;
  const float* srow = a.s + (size_t)row * a.C;
  int32_t* idx = a.idx + (size_t)row * a.kcap;
  float* lg = a.logg != nullptr ? a.logg + (size_t)row * a.kcap : nullptr;

  float x[kSelPer];
  uint32_t key[kSelPer];
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    const int m = m0 + i;
    x[i] = m < n ? srow[m] : -INFINITY;
    if (x[i] != x[i]) x[i] = -INFINITY;
    key[i] = m < n ? order_key(x[i]) : 0u;   // valid keys are >= order_key(-inf) > 0
  }
  float lse = -INFINITY;
  if (a.lse != nullptr || lg != nullptr) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) mx = fmaxf(mx, x[i]);
    mx = block_reduce(mx, red, true);
    if (mx != -INFINITY) {
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < kSelPer; ++i) sum += expf(x[i] - mx);
      sum = block_reduce(sum, red, false);
      lse = mx + logf(sum);
    }
    if (a.lse != nullptr && t == 0) a.lse[row] = lse;
  }

  int need_eq = 0;
  uint32_t T = 0xFFFFFFFFu;   // no block kept when k == 0
  if (k > 0) {
    // Digits of 12, 10 and 10 bits from the top. Scores of one row usually share their
    // sign and a few exponent values, so a wide first digit spreads them over many bins
    // (few LDS atomics collide on one counter).
    uint32_t prefix = 0;
    int remaining = k;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
      const int nbins = pass == 0 ? 4096 : 1024;
      const int hi = shift + (pass == 0 ? 12 : 10);   // bits >= hi are fixed by earlier passes
      const int per = nbins / kSelThreads;             // bins owned by each thread
      for (int i = t; i < nbins; i += kSelThreads) hist[i] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kSelPer; ++i) {
        const bool match = key[i] != 0u && (hi == 32 || (key[i] >> hi) == (prefix >> hi));
        if (match) atomicAdd(&hist[(key[i] >> shift) & (nbins - 1)], 1);
      }
      __syncthreads();
      // thread t owns bins per t .. per t + per - 1; above = matching keys in higher bins
      int local = 0;
      for (int i = 0; i < per; ++i) local += hist[per * t + i];
      int total;
      const int before = block_excl_scan(local, wsum, &total);
      int above = total - before - local;
      for (int i = per - 1; i >= 0; --i) {
        const int c = hist[per * t + i];
        if (above < remaining && remaining <= above + c) {
          pick[0] = per * t + i;
          pick[1] = above;
        }
        above += c;
      }
      __syncthreads();
      prefix |= (uint32_t)pick[0] << shift;
      remaining -= pick[1];
      __syncthreads();   // pick and hist are rewritten by the next pass
    }
    T = prefix;
    need_eq = remaining;   // keys equal to T still to take, lowest index first
  }
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kSelPer; ++i) {
    gt += (key[i] != 0u && key[i] > T);
    eq += (key[i] != 0u && key[i] == T);
  }
  // one scan of both counts (each below 2^14): low 16 bits above-threshold, high 16 ties
  int packed_total;
  const int packed = block_excl_scan(gt | (eq << 16), wsum, &packed_total);
  int gt_before = packed & 0xFFFF, eq_before = packed >> 16;
  if (k > 0) {
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const bool above = key[i] != 0u && key[i] > T;
      const bool tie = key[i] != 0u && key[i] == T;
      if (above || (tie && eq_before < need_eq)) {
        // kept blocks before this one: all blocks above T, the first need_eq ties
        const int pos = gt_before + min(eq_before, need_eq);
        if (pos < k) {   // always true when the threshold is right; keeps writes in the row
          idx[pos] = m0 + i;
          if (lg != nullptr) lg[pos] = (lse == -INFINITY) ? -INFINITY : x[i] - lse;
        }
      }
      gt_before += above;
      eq_before += tie;
    }
  }
  for (int p = k + t; p < a.kcap; p += kSelThreads) {
    idx[p] = -1;
    if (lg != nullptr) lg[p] = 0.0f;
  }
  if (t == 0) a.cnt[row] = k;
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t st) {
  if (a.nblk <= 0) return hipSuccess;
  const dim3 grid((unsigned)((long long)a.B * a.Hkv * a.nblk));
  ProfScope prof("pool", st);
  if (a.d == 128) hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Block scores. Grid: rows x chunks of CH blocks. Each wave reads 64 lanes x 16 bytes =
// BPW pooled keys per load (LPB lanes per key, fully coalesced), NIT loads in flight per
// lane, and reduces each key's partial dot products across its LPB lanes.
template <int D>
__global__ __launch_bounds__(256) void score_kernel(const DecSelArgs a) {
  constexpr int LPB = D / 8, BPW = 64 / LPB, NIT = 8;
  constexpr int CH = 4 * NIT * BPW;
  const int nch = (a.C + CH - 1) / CH;
  const long long row = blockIdx.x / nch;      // (b, h)
  const int chunk = (int)(blockIdx.x % nch);
  const int b = (int)(row / a.Hkv), h = (int)(row % a.Hkv);
  const int hist = min(max((a.kv_len[b] - 1) / kBlock, 0), a.C);
  const int m0 = chunk * CH + (threadIdx.x >> 6) * NIT * BPW;
  if (m0 >= hist) return;   // uniform per wave
  const int lane = threadIdx.x & 63, sub = lane % LPB, bsel = lane / LPB;
  // mean of the group's queries, this lane's 8-element slice
  float qb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* qp = a.q + ((size_t)b * a.Hq + (size_t)h * a.G) * D + 8 * sub;
  for (int g = 0; g < a.G; ++g) {
    const u16x8 v = ld16(qp + (size_t)g * D);
#pragma unroll
    for (int i = 0; i < 8; ++i) qb[i] += bf2f(v[i]);
  }
  const float qs = a.scale / (float)a.G;
  const uint16_t* kp = a.kbar + ((size_t)row * a.C) * D + 8 * sub;
  u16x8 kv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int m = m0 + it * BPW + bsel;
    kv[it] = m < hist ? ld16(kp + (size_t)m * D) : u16x8{};
  }
  float* srow = a.s + (size_t)row * a.C;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) dot += qb[i] * bf2f(kv[it][i]);
#pragma unroll
    for (int o = 1; o < LPB; o <<= 1) dot += __shfl_xor(dot, o, 64);
    const int m = m0 + it * BPW + bsel;
    if (sub == 0 && m < hist) srow[m] = dot * qs;
  }
}

__global__ __launch_bounds__(kSelThreads) void topk_rows_kernel(const DecSelArgs a) {
  __shared__ TopkSmem sm;
  topk_row(a, blockIdx.x, sm);
}

hipError_t launch_decode_select(const DecSelArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.Hkv;
  {
    const int ch = a.d == 128 ? 4 * 8 * 4 : 4 * 8 * 8;
    const long long nch = (a.C + ch - 1) / ch;
    ProfScope prof("block_scores", st);
    if (a.d == 128) hipLaunchKernelGGL(score_kernel<128>, dim3((unsigned)(rows * nch)), dim3(256), 0, st, a);
    else hipLaunchKernelGGL(score_kernel<64>, dim3((unsigned)(rows * nch)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ProfScope prof("topk_rows", st);
  hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(kSelThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sas
