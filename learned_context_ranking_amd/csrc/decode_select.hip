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
#include <type_traits>

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
  const uint16_t* src;
  bool live = true;
  if (a.page_table != nullptr) {   // (uniform per workgroup)
    const int pg = a.page_table[(size_t)b * a.C + m];
    live = pg >= 0 && pg < a.num_pages;
    src = a.K + ((size_t)(live ? pg : 0) * a.Hkv + (size_t)(bh % a.Hkv)) * kBlock * D + 8 * c;
  } else {
    src = a.K + ((size_t)bh * a.Lmax + (size_t)m * kBlock) * D + 8 * c;
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (live) {
#pragma unroll
    for (int r = rg; r < kBlock; r += RG) {
      const u16x8 v = ld16(src + (size_t)r * D);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += bf2f(v[i]);
    }
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
static_assert(kMaxCols == 32 * kSelThreads, "each thread owns 32 consecutive blocks of a row");

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
  v = is_max ? dpp_max(v) : dpp_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kSelThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

// Top-K of one row by one workgroup. The row's order keys are staged in LDS; the K-th
// largest is found digit by digit (passes of 12, 10 and 10 bits over an LDS histogram of
// the keys that match the digits fixed so far), stopping early once the chosen bin holds
// exactly the places still open. Keys above the cut are kept and the remaining places go
// to the lowest-index keys at the cut. Every loop runs over the row's actual length, and
// LDS arrays are padded (one word per 32 keys, one per bin group) so the strided and the
// per-thread-contiguous accesses are both free of bank conflicts.
constexpr int kKeyPad = kMaxCols + kMaxCols / 32;
struct TopkSmem {
  uint32_t keys[kKeyPad];
  int hist[4096 + 256];
  int wsum[kSelThreads / 64];
  float red[kSelThreads / 64];
  int pick[3];
};

__device__ __forceinline__ int kpad(int m) { return m + (m >> 5); }
__device__ __forceinline__ float key_value(uint32_t k) {   // inverse of order_key
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ void topk_row(const DecSelArgs& a, long long row, TopkSmem& sm) {
  int* hist = sm.hist;
  const int b = (int)(row / a.Hkv);
  const int n = min(max((a.kv_len[b] - 1) / kBlock, 0), a.C);
  const int k = min(a.topk, n);
  const int t = threadIdx.x;
  const float* srow = a.s + (size_t)row * a.C;
  int32_t* idx = a.idx + (size_t)row * a.kcap;
  float* lg = a.logg != nullptr ? a.logg + (size_t)row * a.kcap : nullptr;

#pragma unroll 8
  for (int m = t; m < n; m += kSelThreads) sm.keys[kpad(m)] = order_key(srow[m]);   // coalesced
  __syncthreads();
  float lse = -INFINITY;
  if (a.lse != nullptr || lg != nullptr) {
    float mx = -INFINITY;
#pragma unroll 8
    for (int m = t; m < n; m += kSelThreads) mx = fmaxf(mx, key_value(sm.keys[kpad(m)]));
    mx = block_reduce(mx, sm.red, true);
    if (mx != -INFINITY) {
      float sum = 0.0f;
#pragma unroll 8
      for (int m = t; m < n; m += kSelThreads) sum += expf(key_value(sm.keys[kpad(m)]) - mx);
      sum = block_reduce(sum, sm.red, false);
      lse = mx + logf(sum);
    }
    if (a.lse != nullptr && t == 0) a.lse[row] = lse;
  }

  // the cut: keys whose bits above cut_shift exceed those of T are kept, and need_eq of
  // the keys equal to T there (lowest index first)
  uint32_t T = 0xFFFFFFFFu;
  int cut_shift = 0, need_eq = 0;
  if (k > 0) {
    uint32_t prefix = 0;
    int remaining = k;
    // one pass over bits [SHIFT, SHIFT + log2 NB) of the keys that match prefix above HI;
    // returns true once the chosen bin holds exactly the places still open
    auto pass = [&](auto shift_c, auto nbins_c, auto hi_c) {
      constexpr int SHIFT = decltype(shift_c)::value, NB = decltype(nbins_c)::value;
      constexpr int HI = decltype(hi_c)::value, PER = NB / kSelThreads;
      // bin b lives at b + b / PER: thread t's bins are contiguous and threads are PER + 1
      // words apart (odd), so neither the strided zeroing nor the per-thread reads collide
#pragma unroll
      for (int i = 0; i < PER; ++i) hist[(PER + 1) * t + i] = 0;
      __syncthreads();
#pragma unroll 8
      for (int m = t; m < n; m += kSelThreads) {
        const uint32_t key = sm.keys[kpad(m)];
        if (HI == 32 || (key >> (HI & 31)) == (prefix >> (HI & 31))) {
          const int bin = (int)((key >> SHIFT) & (uint32_t)(NB - 1));
          atomicAdd(&hist[bin + bin / PER], 1);
        }
      }
      __syncthreads();
      int c[PER];
      int local = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        c[i] = hist[(PER + 1) * t + i];
        local += c[i];
      }
      int total;
      const int before = block_excl_scan(local, sm.wsum, &total);
      int above = total - before - local;   // matching keys in higher bins
#pragma unroll
      for (int i = PER - 1; i >= 0; --i) {
        if (above < remaining && remaining <= above + c[i]) {
          sm.pick[0] = PER * t + i;
          sm.pick[1] = above;
          sm.pick[2] = c[i];
        }
        above += c[i];
      }
      __syncthreads();
      prefix |= (uint32_t)sm.pick[0] << SHIFT;
      remaining -= sm.pick[1];
      const int in_bin = sm.pick[2];
      __syncthreads();   // pick and hist are rewritten by the next pass
      cut_shift = SHIFT;
      return in_bin == remaining;
    };
    using I = int;
    if (!pass(std::integral_constant<I, 20>{}, std::integral_constant<I, 4096>{}, std::integral_constant<I, 32>{}))
      if (!pass(std::integral_constant<I, 10>{}, std::integral_constant<I, 1024>{}, std::integral_constant<I, 20>{}))
        pass(std::integral_constant<I, 0>{}, std::integral_constant<I, 1024>{}, std::integral_constant<I, 10>{});
    T = prefix;
    need_eq = remaining;
  }
  // thread t counts and then writes blocks 32 t .. 32 t + 31 (index order); the key reads
  // are unrolled so they are in flight together
  const int m0 = 32 * t;
  uint32_t kk[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) kk[i] = (k > 0 && m0 + i < n) ? sm.keys[kpad(m0 + i)] : 0u;   // 0: no block
  const uint32_t tc = T >> cut_shift;
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    gt += kk[i] != 0u && (kk[i] >> cut_shift) > tc;
    eq += kk[i] != 0u && (kk[i] >> cut_shift) == tc;
  }
  // one scan of both counts (each below 2^14): low 16 bits above the cut, high 16 at it
  int packed_total;
  const int packed = block_excl_scan(gt | (eq << 16), sm.wsum, &packed_total);
  int gt_before = packed & 0xFFFF, eq_before = packed >> 16;
  if (gt + eq > 0) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const bool above = kk[i] != 0u && (kk[i] >> cut_shift) > tc;
      const bool tie = kk[i] != 0u && (kk[i] >> cut_shift) == tc;
      if (above || (tie && eq_before < need_eq)) {
        // kept blocks before this one: all blocks above the cut, the first need_eq ties
        const int pos = gt_before + min(eq_before, need_eq);
        if (pos < k) {   // always true when the cut is right; keeps writes in the row
          idx[pos] = m0 + i;
          if (lg != nullptr) lg[pos] = (lse == -INFINITY) ? -INFINITY : key_value(kk[i]) - lse;
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

// Block scores of one wave: NIT loads of 64 lanes x 16 bytes = BPW pooled keys each (LPB
// lanes per key, fully coalesced, all NIT in flight), each key's partial dot products
// reduced across its LPB lanes. f(m, score) is called, on one lane per key, for the wave's
// blocks m0 .. m0 + NIT * BPW - 1 below hist.
template <int D>
struct WaveScores {
  static constexpr int LPB = D / 8, BPW = 64 / LPB, NIT = 8, PER_WAVE = NIT * BPW;
  float qb[8];   // mean of the group's queries (this lane's 8-element slice), times scale / G
  __device__ __forceinline__ WaveScores(const DecSelArgs& a, int b, int h) {
    const int sub = (threadIdx.x & 63) % LPB;
#pragma unroll
    for (int i = 0; i < 8; ++i) qb[i] = 0.0f;
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + (size_t)h * a.G) * D + 8 * sub;
    for (int g = 0; g < a.G; ++g) {
      const u16x8 v = ld16(qp + (size_t)g * D);
#pragma unroll
      for (int i = 0; i < 8; ++i) qb[i] += bf2f(v[i]);
    }
  }
  template <class F>
  __device__ __forceinline__ void run(const DecSelArgs& a, long long row, int m0, int hist, F&& f) const {
    const int lane = threadIdx.x & 63, sub = lane % LPB, bsel = lane / LPB;
    const float qs = a.scale / (float)a.G;
    const uint16_t* kp = a.kbar + ((size_t)row * a.C) * D + 8 * sub;
    u16x8 kv[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int m = m0 + it * BPW + bsel;
      kv[it] = m < hist ? ld16(kp + (size_t)m * D) : u16x8{};
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot += qb[i] * bf2f(kv[it][i]);
#pragma unroll
      for (int o = 1; o < LPB; o <<= 1) dot += __shfl_xor(dot, o, 64);
      const int m = m0 + it * BPW + bsel;
      if (sub == 0 && m < hist) f(m, dot * qs);
    }
  }
};

// Block scores. Grid: rows x chunks of 4 waves x PER_WAVE blocks.
template <int D>
__global__ __launch_bounds__(256) void score_kernel(const DecSelArgs a) {
  using W = WaveScores<D>;
  constexpr int CH = 4 * W::PER_WAVE;
  const int nch = (a.C + CH - 1) / CH;
  const long long row = blockIdx.x / nch;      // (b, h)
  const int chunk = (int)(blockIdx.x % nch);
  const int b = (int)(row / a.Hkv), h = (int)(row % a.Hkv);
  const int hist = min(max((a.kv_len[b] - 1) / kBlock, 0), a.C);
  const int m0 = chunk * CH + (threadIdx.x >> 6) * W::PER_WAVE;
  if (m0 >= hist) return;   // uniform per wave
  const W ws(a, b, h);
  float* srow = a.s + (size_t)row * a.C;
  ws.run(a, row, m0, hist, [&](int m, float v) { srow[m] = v; });
}

// Candidates: the scores of a chunk of CH = R x 4 x PER_WAVE blocks (each wave R runs of
// the scoring above) go to LDS, and one wave keeps the chunk's min(K, blocks) best by the
// selection's own search and walk (order keys: NaN as -inf, -0 as +0; ties to the lower
// block). Every block of the row's global Top-K is among its chunk's K best, so the Top-K
// of the candidates is the Top-K of the row; the slots keep ascending block order, so a
// tie between candidates still goes to the lower block. Every slot of the chunk is
// written (empty ones: block -1, score 0), also for chunks past the row's history.
template <int D, int R>
__global__ __launch_bounds__(256) void cand_kernel(const DecSelArgs a) {
  using W = WaveScores<D>;
  constexpr int CH = R * 4 * W::PER_WAVE, PL = CH / 64;
  __shared__ float sc[CH];
  const int nch = (a.C + CH - 1) / CH;
  const long long row = blockIdx.x / nch;
  const int chunk = (int)(blockIdx.x % nch);
  const int b = (int)(row / a.Hkv), h = (int)(row % a.Hkv);
  // (kv_len is clamped to the cache as the decode clamps it, so both see the same history)
  const int hist = min(max((a.kv_len[b] - 1) / kBlock, 0), min(a.C, a.hist_cap));
  const int base = chunk * CH;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (base < hist) {
    const W ws(a, b, h);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int m0 = base + (r * 4 + wv) * W::PER_WAVE;
      if (m0 < hist) ws.run(a, row, m0, hist, [&](int m, float v) { sc[m - base] = v; });
    }
  }
  __syncthreads();
  if (wv != 0) return;
  const int valid = min(max(hist - base, 0), CH);   // the chunk's history blocks (uniform)
  const int k = min(a.topk, valid);
  float* cs = a.cs + (size_t)row * a.cld + (size_t)chunk * a.topk;
  int32_t* ci = a.ci + (size_t)row * a.cld + (size_t)chunk * a.topk;
  for (int p = k + lane; p < a.topk; p += 64) { cs[p] = 0.0f; ci[p] = -1; }
  if (k == 0) return;
  const int nreg = (valid + 63) >> 6;
  uint32_t key[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    float v = lane + 64 * i < valid ? sc[lane + 64 * i] : 0.0f;
    v = v == v ? v : -INFINITY;   // NaN ranks as -inf
    v = v == 0.0f ? 0.0f : v;     // -0 equals +0
    key[i] = lane + 64 * i < valid ? sas::order_key(v) : 0u;
  }
  uint32_t T;
  int need_eq;
  topk_cut(key, nreg, valid, k, T, need_eq);
  topk_walk(key, nreg, T, need_eq, [&](int i, int pos) {
    cs[pos] = sc[lane + 64 * i];
    ci[pos] = base + lane + 64 * i;
  });
}

int decode_cand_chunk(int C, int topk, int d) {
  const int per = 4 * (d == 128 ? WaveScores<128>::PER_WAVE : WaveScores<64>::PER_WAVE);
  for (int ch = per; ch <= 1024; ch *= 2)   // (a chunk is ranked by one wave, <= 16 keys a lane)
    if ((long long)((C + ch - 1) / ch) * topk <= kDecSelMaxCols) return ch;
  return 0;   // more slots than one decode row ranks
}

hipError_t launch_decode_candidates(const DecSelArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.Hkv;
  const dim3 grid((unsigned)(rows * ((a.C + a.cch - 1) / a.cch)));
  const int r = a.cch / (4 * (a.d == 128 ? WaveScores<128>::PER_WAVE : WaveScores<64>::PER_WAVE));
  ProfScope prof("decode_candidates", st);
  if (a.d == 128) {
    if (r == 1) hipLaunchKernelGGL((cand_kernel<128, 1>), grid, dim3(256), 0, st, a);
    else if (r == 2) hipLaunchKernelGGL((cand_kernel<128, 2>), grid, dim3(256), 0, st, a);
    else if (r == 4) hipLaunchKernelGGL((cand_kernel<128, 4>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((cand_kernel<128, 8>), grid, dim3(256), 0, st, a);
  } else {
    if (r == 1) hipLaunchKernelGGL((cand_kernel<64, 1>), grid, dim3(256), 0, st, a);
    else if (r == 2) hipLaunchKernelGGL((cand_kernel<64, 2>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((cand_kernel<64, 4>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

__global__ __launch_bounds__(kSelThreads) void topk_rows_kernel(const DecSelArgs a) {
  __shared__ TopkSmem sm;
  topk_row(a, blockIdx.x, sm);
}

hipError_t launch_decode_select(const DecSelArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.Hkv;
  {
    const int ch = 4 * (a.d == 128 ? WaveScores<128>::PER_WAVE : WaveScores<64>::PER_WAVE);
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
