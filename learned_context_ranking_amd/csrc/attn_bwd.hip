// Backward of log-gated block-sparse attention, with the gate gradient (gfx950).
//
// Content gradients are those of softmax attention over S_j; only attended keys receive
// them (sparse scope, [SAS-ko] "무엇과 다른가", choice 4). The gate gradient follows choice 1
// of the same section: dg_jm = sum_{t, i in B_m} (p~_ti / g_jm) dO_t.(v_i - o_t), summed
// over the G * 64 query rows that share the selection. Since p~_ti / g_jm =
// exp(scale q_t.k_i - LSE_t) (eq. (9) of [SAS-ja] "仕組み"), each tile accumulates
// u_ti * (dP_ti - delta_t) with u the ungated weight; this stays exact when g is tiny.
//
// Passes (no atomics, deterministic):
//   1. inverse index: for every key block m, the ascending list of (j, slot) with
//      idx[j][slot] = m, found by binary search in the ascending idx rows; the lists of
//      one (b, KV head) live in its own NB * kcap slice of the list buffer. The scan of
//      the list lengths also plans pass 3: lists too long for one workgroup (with skewed
//      scores some key blocks are selected by nearly every later query block) are cut
//      into segments, and the segments are ordered longest first
//   2. query-major pass, one workgroup per (b, KV head, j, pair of query heads): delta_t =
//      dO_t . o_t for its rows, dQ, and the workgroup's share of dg. Each dg_jm is owned by
//      the workgroups of query block j; their per-split partials are summed in a fixed
//      order by a small reduction kernel. Per row it also stores -delta_t and
//      -LSE_t / scale, the start values of the key-major pass's dP and S accumulators
//   3. key-major pass, one workgroup per planned segment of (b, KV head, m): dK and dV over
//      the current block m itself plus every query block that selected m, for all G heads.
//      The first segment of a block writes its rows of dK / dV, later ones a partial slot;
//      a small kernel adds the partials in segment order
//
// All 64-row operand tiles live in LDS in the swizzled layout of Tile<D>, copied straight
// from global memory (global_load_lds) one block ahead of use. Operands whose contraction
// runs along the rows of a tile (K^T for dQ, Q^T and dO^T for dK and dV) are read with the
// transposing ds_read_b64_tr_b16 from the same natural tile.
#include <algorithm>

#include <type_traits>

#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

constexpr int kDkvMinSeg = 64;   // shortest segment (items) a key block's list is cut into

// ---------------------------------------------------------------- small kernels

__global__ void fill_f32_kernel(float* p, long long n, float v) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

// Number of the valid selection entries of rows j > m that name block m.
__device__ __forceinline__ int find_in_row(const int32_t* row, int n, int m) {
  int lo = 0, hi = n - 1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int v = row[mid];
    if (v == m) return mid;
    if (v < m) lo = mid + 1; else hi = mid - 1;
  }
  return -1;
}

// One wave per (b, h, m): scan query blocks j > m; with `list` == nullptr only count.
__global__ __launch_bounds__(256) void inv_kernel(const int32_t* idx, const int32_t* cnt, int NB,
                                                  int kcap, long long nrows, int32_t* counts,
                                                  const int32_t* off, int32_t* list) {
  const int lane = threadIdx.x & 63;
  const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= nrows) return;
  const int m = (int)(w % NB);
  const long long bh = w / NB;
  const int32_t* idx_bh = idx + bh * NB * kcap;
  const int32_t* cnt_bh = cnt + bh * NB;
  int base = 0;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int32_t* out = list != nullptr ? list + bh * NB * kcap + off[bh * (NB + 1) + m] : nullptr;
  for (int j0 = m + 1; j0 < NB; j0 += 64) {
    const int j = j0 + lane;
    int slot = -1;
    if (j < NB) {
      const int c = min(max(cnt_bh[j], 0), min(kcap, j));
      slot = find_in_row(idx_bh + (long long)j * kcap, c, m);
    }
    const unsigned long long bal = __ballot(slot >= 0);
    if (out != nullptr && slot >= 0) out[base + __popcll(bal & lt)] = j * kcap + slot;
    base += __popcll(bal);
  }
  if (list == nullptr && lane == 0) counts[w] = base;
}

// Exclusive scan of one value per thread of a 256-thread block (4 waves); *total receives
// the sum. red4 is 4 ints of LDS.
__device__ __forceinline__ int scan256(int32_t* red4, int v, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) red4[w] = x;
  __syncthreads();
  int before = 0;
  for (int u = 0; u < w; ++u) before += red4[u];
  *total = (red4[0] + red4[1]) + (red4[2] + red4[3]);
  __syncthreads();
  return before + x - v;
}

// Sum / maximum over a 256-thread block (every thread gets the result).
__device__ __forceinline__ int block_sum256(int32_t* red4, int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = v;
  __syncthreads();
  const int r = (red4[0] + red4[1]) + (red4[2] + red4[3]);
  __syncthreads();
  return r;
}
__device__ __forceinline__ int block_max256(int32_t* red4, int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = v;
  __syncthreads();
  const int r = max(max(red4[0], red4[1]), max(red4[2], red4[3]));
  __syncthreads();
  return r;
}

// Length class of a segment for the longest-first order: 4 classes per octave.
__device__ __forceinline__ int len_class(int len) {
  len = max(len, 1);
  const int lg = 31 - __clz(len);
  return min(63, lg < 2 ? len : 4 * lg + ((len >> (lg - 2)) & 3));
}

// Per (b, h), one workgroup: the exclusive scan of the per-block counts, off[0..NB], and
// the key-major pass's work plan. Key block m has items_m = (count_m + 1) * G (its list and
// itself, for each of the G heads). A list longer than the segment length T is cut into
// nseg_m = ceil(items_m / T) segments, one workgroup each; T is the smallest length >=
// kDkvMinSeg for which the extra segments fit the budget of partial-result slots. seg_tab
// lists the segments of (b, h) as {m, s, nseg_m, partial slot (-1 for s = 0)}, longest first
// by length class and in key-block order within a class (a fixed order: the plan does not
// depend on timing), then {-1, ...} up to NB + budget entries; red_tab lists the split
// blocks as {m, nseg_m, first partial slot, 0}, then {-1, ...} up to budget entries.
__global__ __launch_bounds__(256) void inv_scan_kernel(const int32_t* counts, int NB, int G, int budget,
                                                       int32_t* off, int4* seg_tab, int4* red_tab) {
  constexpr int NCLS = 64, PITCH = 260;   // hist row: one column per thread, padded
  __shared__ int32_t red4[4];
  __shared__ int32_t hist[NCLS * PITCH];   // [class][thread]: segments, then positions
  const long long bh = blockIdx.x;
  const int per = (NB + 255) / 256;
  const int t = threadIdx.x;
  const int i0 = min(NB, t * per), i1 = min(NB, (t + 1) * per);
  const int32_t* cnt = counts + bh * NB;
  int s = 0, mx = 0;
  for (int i = i0; i < i1; ++i) {
    s += cnt[i];
    mx = max(mx, (cnt[i] + 1) * G);
  }
  int tot;
  int run = scan256(red4, s, &tot);
  for (int i = i0; i < i1; ++i) {
    off[bh * (NB + 1) + i] = run;
    run += cnt[i];
  }
  if (t == 255) off[bh * (NB + 1) + NB] = run;

  // segment length by bisection (uniform: every thread sees the same sums)
  const int maxItems = block_max256(red4, mx);
  int lo = kDkvMinSeg, hi = max(kDkvMinSeg, maxItems);
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    int ex = 0;
    for (int i = i0; i < i1; ++i) ex += ((cnt[i] + 1) * G + mid - 1) / mid - 1;
    if (block_sum256(red4, ex) <= budget) hi = mid; else lo = mid + 1;
  }
  const int T = lo;
  auto nseg_of = [&](int i) { return ((cnt[i] + 1) * G + T - 1) / T; };
  auto seg_len = [&](int i, int q, int k) {
    const int all = (cnt[i] + 1) * G, ts = (all + q - 1) / q;
    return k < q - 1 ? ts : all - (q - 1) * ts;
  };
  // position of each segment: classes from the longest down, then thread (key block) order
  for (int c = 0; c < NCLS; ++c) hist[c * PITCH + t] = 0;
  int nx = 0, nr = 0;
  for (int i = i0; i < i1; ++i) {
    const int q = nseg_of(i);
    nx += q - 1;
    nr += q > 1;
    for (int k = 0; k < q; ++k) ++hist[(NCLS - 1 - len_class(seg_len(i, q, k))) * PITCH + t];
  }
  __syncthreads();
  {
    // thread t scans the 64 entries [64 t, 64 t + 64) of the class-major order in place
    const int c = t >> 2, u0 = (t & 3) * 64;
    int32_t* h = hist + c * PITCH + u0;
    int sum = 0;
    for (int u = 0; u < 64; ++u) sum += h[u];
    int nsegs;
    int base = scan256(red4, sum, &nsegs);
    for (int u = 0; u < 64; ++u) {
      const int x = h[u];
      h[u] = base;
      base += x;
    }
    __syncthreads();
    const int slots = NB + budget;
    int4* st = seg_tab + bh * slots;
    int4* rt = red_tab + bh * budget;
    int nred;
    int xo = scan256(red4, nx, &tot);
    int ro = scan256(red4, nr, &nred);
    const int pbase = (int)bh * budget;
    for (int i = i0; i < i1; ++i) {
      const int q = nseg_of(i);
      for (int k = 0; k < q; ++k) {
        const int pos = hist[(NCLS - 1 - len_class(seg_len(i, q, k))) * PITCH + t]++;
        st[pos] = make_int4(i, k, q, k == 0 ? -1 : pbase + xo + k - 1);
      }
      if (q > 1) rt[ro++] = make_int4(i, q, pbase + xo, 0);
      xo += q - 1;
    }
    for (int k = nsegs + t; k < slots; k += 256) st[k] = make_int4(-1, 0, 0, 0);
    for (int k = nred + t; k < budget; k += 256) rt[k] = make_int4(-1, 0, 0, 0);
  }
}

// Sum of the partial dK / dV of the split key blocks, in segment order: the first segment
// wrote the block's rows of dK / dV directly; segments 1 .. nseg - 1 their partial slots.
template <int D>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(const int4* red_tab, int budget, int n,
                                                         const float* part, float* dK, float* dV) {
  const long long bh = blockIdx.x / budget;
  const int4 e = red_tab[blockIdx.x];
  if (e.x < 0) return;
  const size_t rows = ((size_t)bh * n + (size_t)e.x * kBlock) * D;
  // 16-byte accesses; the partials of four segments are loaded together, then added in
  // segment order (the result does not depend on the grouping)
  constexpr int N4 = kBlock * D / 4;
  const f32x4* pp = reinterpret_cast<const f32x4*>(part) + (size_t)e.z * (2 * N4);
  for (int i = threadIdx.x; i < N4; i += 256) {
    f32x4 k = reinterpret_cast<const f32x4*>(dK + rows)[i];
    f32x4 v = reinterpret_cast<const f32x4*>(dV + rows)[i];
    int sgm = 1;
    for (; sgm + 4 <= e.y; sgm += 4) {
      f32x4 pk[4], pv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4* p = pp + (size_t)(sgm - 1 + u) * (2 * N4);
        pk[u] = p[i];
        pv[u] = p[N4 + i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) { k += pk[u]; v += pv[u]; }
    }
    for (; sgm < e.y; ++sgm) {
      const f32x4* p = pp + (size_t)(sgm - 1) * (2 * N4);
      k += p[i];
      v += p[N4 + i];
    }
    reinterpret_cast<f32x4*>(dK + rows)[i] = k;
    reinterpret_cast<f32x4*>(dV + rows)[i] = v;
  }
}

// ---------------------------------------------------------------- query-major: dQ, dg

// 4 waves: 2 query heads x 2 halves of the 64 query rows (32 rows per wave). When G is
// odd the last split has one head; the waves of the missing head take part in the copies
// and barriers only.
// The K/V blocks stream through two LDS buffer sets (distinct objects selected at compile
// time); block t+1 is copied in (buffer loads into LDS with a scalar per-block offset)
// while block t is computed. The copy is issued on every step, past the end of the list it
// repeats the last block, so the compiler's wait tracking stays exact.
template <int D, bool OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(const AttnArgs a, int nsplit) {
  constexpr int NW = 4;
  __shared__ __attribute__((aligned(16))) uint16_t sk0[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[Tile<D>::ELEMS];
  __shared__ float dgp[2][4];   // per-wave dg partials of the last two blocks
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5, ql = lane & 31;
  const int NB = a.n / kBlock, G = a.Hq / a.Hkv;
  const int BH = a.B * a.Hkv;
  const int per_j = BH * nsplit;
  const unsigned bid = wg_index(a.wg);
  const int j = NB - 1 - (int)(bid / per_j);
  const int r = bid % per_j;
  const int split = r / BH;
  const int h = (r % BH) % a.Hkv, b = (r % BH) / a.Hkv;
  const int head0 = split * 2;
  const int nheads = min(2, G - head0);
  const int whead = wave >> 1, wrow0 = (wave & 1) * 32;
  const bool active = whead < nheads;
  const int hq = h * G + head0 + (active ? whead : 0);

  const size_t kv_off = ((size_t)(b * a.Hkv + h) * a.n) * D;
  const size_t row_off = (size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock + wrow0;
  const size_t q_off = row_off * D;
  const size_t sel_row = (size_t)(b * a.Hkv + h) * NB + j;
  const int cnt_j = min(max(a.cnt[sel_row], 0), min(a.kcap, j));
  const int32_t* idx_row = a.idx + sel_row * a.kcap;
  const float* lg_row = a.logg != nullptr ? a.logg + sel_row * a.kcap : nullptr;
  float* dg_out = (nsplit == 1 ? a.dg : a.dg_part + (size_t)split * BH * NB * a.kcap) + sel_row * a.kcap;

  // Q and dO as B operands (query ql, d = 16 ks + 8 hl + e); delta = dO . O for the same rows
  bf16x8 qf[D / 16], dof[D / 16];
  float dlt = 0.0f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const size_t o = q_off + ql * D + 16 * ks + 8 * hl;
    qf[ks] = as_bf16x8(ld16(a.Q + o));
    dof[ks] = as_bf16x8(ld16(a.dO + o));
    const u16x8 ov = ld16(a.O + o);
#pragma unroll
    for (int e = 0; e < 8; ++e) dlt += bf2f(ov[e]) * (float)dof[ks][e];
  }
  dlt = half_sum(dlt);
  const float lse = a.lse_rows[row_off + ql];
  if (active && hl == 0) {
    a.ndelta[row_off + ql] = -dlt;
    a.nlse[row_off + ql] = -lse / a.scale;
  }
  const float lse2 = lse * kLog2e;

  // per-lane byte offsets of this wave's 16-byte slots within a 64-row tile
  constexpr int NWIN = Tile<D>::CPR / NW;
  uint32_t voff[NWIN];
#pragma unroll
  for (int i = 0; i < NWIN; ++i) {
    const int sidx = 64 * (wave + NW * i) + lane;
    const int rr = sidx / Tile<D>::CPR, c = sidx % Tile<D>::CPR;
    voff[i] = (uint32_t)(rr * D + ((c ^ Tile<D>::swz(rr)) << 3)) * 2u;
  }
  const uint16_t* kbase = a.K + kv_off;
  const uint16_t* vbase = a.V + kv_off;
  const int kvbytes = a.n * D * 2;

  // Block t of the list: t = 0 is block j itself, t >= 1 the selected block idx[t - 1].
  // (tc: block being computed; tf: next block to copy, which stays at cnt_j once reached.)
  auto load_sel = [&](int i, int& v, float& g) {
    v = i < cnt_j ? idx_row[i] : 0;
    g = (i < cnt_j && lg_row != nullptr) ? lg_row[i] * kLog2e : 0.0f;
  };
  LaneList sel_c, sel_f;
  int tc = 0, tf = 0;
  auto fetch = [&](uint16_t* kb, uint16_t* vb) {
    int mb = j;
    if (tf > 0) {
      sel_f.ensure(tf - 1, lane, load_sel);
      mb = sel_f.at(tf - 1);
      if (mb < 0 || mb >= j) mb = 0;
    }
    const uint32_t so = (uint32_t)mb * (uint32_t)(kBlock * D * 2);
#pragma unroll
    for (int i = 0; i < NWIN; ++i) buffer_load_lds16(kbase, kvbytes, kb + 512 * (wave + NW * i), voff[i], so);
#pragma unroll
    for (int i = 0; i < NWIN; ++i) buffer_load_lds16(vbase, kvbytes, vb + 512 * (wave + NW * i), voff[i], so);
    if (tf < cnt_j) ++tf;
  };

  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[dt][i] = 0.0f;
  const float c2 = a.scale * kLog2e;
  const int g16 = lane >> 4, lp = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (lp >> 2), tr_d = 16 * (g16 & 1) + 4 * (lp & 3);
  // Lane base offsets (elements) in the Tile layout: row read ks of key row 32 mt + ql at
  // d = 16 ks + 8 hl sits at 32 mt D + (rx ^ (ks << 4)); the transposing read of rows
  // r0 + tr_row (r0 = 32 mt + 16 hh + 8 half) at d = 32 dt + tr_d at
  // r0 D + (tx ^ ((4 dt ^ 2 half) << 3)).
  const int rx0 = ql * D + ((hl ^ Tile<D>::swz(ql)) << 3);
  const int tx0 = tr_row * D + ((((tr_d >> 3) ^ Tile<D>::swz(tr_row))) << 3) + (tr_d & 7);

  // one block: copy the next block into (kn, vn), compute block tc from (kc, vc)
  // DIAG: the step of block t = 0 (block j itself), the only one with a causal mask; it is
  // peeled off the loop so the other steps carry no masking code
  auto step = [&](auto diag_c, const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    constexpr bool DIAG = decltype(diag_c)::value;
    wait_vm();
    barrier_lds();
    const int t = tc;
    float lg2 = 0.0f;
    bool ok = true;
    if (!DIAG) {
      sel_c.ensure(t - 1, lane, load_sel);
      const int mb = sel_c.at(t - 1);
      lg2 = sel_c.gat(t - 1);
      if (mb < 0 || mb >= j) { lg2 = -INFINITY; ok = false; }
    }
    ++tc;
    fetch(kn, vn);
    // dg of the previous block: sum of the four waves' partials
    if (t >= 2 && tid == 0) {
      const float* pp = dgp[(t - 1) & 1];
      dg_out[t - 2] = (pp[0] + pp[1]) + (pp[2] + pp[3]);
    }
    if (!active) {   // a missing head's waves only take part in the copies
      if (lane == 0) dgp[t & 1][wave] = 0.0f;
      return;
    }
    float dgacc = 0.0f;
    const float g = fast_exp2(lg2);
    int rx = rx0, tx = tx0;
    asm volatile("" : "+v"(rx), "+v"(tx));   // keeps per-(buffer, read) addresses unhoisted
    // The two 32-key halves of the block one after the other; the scheduling barriers bound
    // how many operand reads are in flight (registers are tight at 2 waves per SIMD).
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 st = {}, dpt = {};
#pragma unroll
      for (int k0 = 0; k0 < D / 16; k0 += 4) {
        bf16x8 kr[4], vr[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int o = 32 * mt * D + (rx ^ ((k0 + u) << 4));
          kr[u] = as_bf16x8(ld16(&kc[o]));
          vr[u] = as_bf16x8(ld16(&vc[o]));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          st = mfma32(kr[u], qf[k0 + u], st);
          dpt = mfma32(vr[u], dof[k0 + u], dpt);
        }
      }
      // K^T operands of dQ^T += K^T dS^T over these 32 keys, read while the softmax runs
      bf16x8 ka[D / 32][2];
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r0 = 32 * mt + 16 * hh;
          ka[dt][hh] = join_tr16(lds_tr16(&kc[r0 * D + (tx ^ ((4 * dt) << 3))]),
                                 lds_tr16(&kc[(r0 + 8) * D + (tx ^ ((4 * dt ^ 2) << 3))]));
        }
      bf16x8 dsf[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float ds[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int i = 8 * hh + x;
          float u = fast_exp2(st[i] * c2 - lse2);   // p~ / g = exp(scale q.k - LSE)
          const int key = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (DIAG && key > wrow0 + ql) u = 0.0f;   // causal mask of block j itself
          if (OUT) {
            // gate after the softmax: u is the probability itself (LSE of the ungated
            // logits); dS = u (g dP - delta), dg = sum u dP; a block outside S has u = 0
            if (!ok) u = 0.0f;
            dgacc += u * dpt[i];
            ds[x] = u * (g * dpt[i] - dlt);
          } else {
            const float w = u * (dpt[i] - dlt);
            dgacc += w;
            ds[x] = w * g;
          }
        }
        dsf[hh] = pack8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) dq[dt] = mfma32(ka[dt][hh], dsf[hh], dq[dt]);
    }
    dgacc = dpp_sum(dgacc);
    if (lane == 0) dgp[t & 1][wave] = (!DIAG && ok) ? dgacc : 0.0f;
  };
  const std::integral_constant<bool, true> diag_step;
  const std::integral_constant<bool, false> plain_step;
  const int nrest = cnt_j;   // steps after the diagonal one
  const int nfull = nrest & ~1;
  fetch(sk0, sv0);
  step(diag_step, sk0, sv0, sk1, sv1);
  for (int it = 0; it < nfull; it += 2) {
    step(plain_step, sk1, sv1, sk0, sv0);
    step(plain_step, sk0, sv0, sk1, sv1);
  }
  if (nfull < nrest) step(plain_step, sk1, sv1, sk0, sv0);
  wait_vm();
  __syncthreads();
  if (tid == 0) {
    if (cnt_j >= 1) {
      const float* pp = dgp[cnt_j & 1];
      dg_out[cnt_j - 1] = (pp[0] + pp[1]) + (pp[2] + pp[3]);
    }
    for (int p = cnt_j; p < a.kcap; ++p) dg_out[p] = 0.0f;
  }
  if (!active) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * dt + 8 * g4 + 4 * hl;
      f32x4 v;
      v[0] = dq[dt][4 * g4 + 0] * a.scale;
      v[1] = dq[dt][4 * g4 + 1] * a.scale;
      v[2] = dq[dt][4 * g4 + 2] * a.scale;
      v[3] = dq[dt][4 * g4 + 3] * a.scale;
      *reinterpret_cast<f32x4*>(a.dQ + q_off + ql * D + d0) = v;
    }
}

// Sum of the per-split dg partials in split order (deterministic).
__global__ void dg_reduce_kernel(const float* part, float* dg, long long n, int nsplit) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int k = 0; k < nsplit; ++k) s += part[(long long)k * n + i];
    dg[i] = s;
  }
}

// ---------------------------------------------------------------- key-major: dK, dV

// Key-major pass, four waves per (b, KV head, key block m) segment and two workgroups per
// CU: wave w owns keys 16 w .. 16 w + 15 of block m and every one of the 64 query rows of
// each item, so its dK / dV rows are complete when the list ends (no reduction across
// waves) and its registers stay within the budget of two waves per SIMD. The two
// workgroups on a CU run independent items: one wave's softmax overlaps the other's
// matrix products.
//
// Products (16x16x32 bf16 MFMAs, fp32 accumulate), per item and wave:
//   S  = Q K^T   (64 rows x 16 keys): A = Q rows from LDS, B = K from registers
//   dP = dO V^T  (64 rows x 16 keys): A = dO rows from LDS, B = V from registers
//   dV^T += dO^T P, dK^T += Q^T dS   (d x 16 keys, contraction over the 64 rows)
// A lane of the S / dP accumulators holds one key and 16 rows {16 rt + 4 u + i}; for the
// contraction over rows the MFMA's k order is taken as a permutation of the rows
// (position 8 u + x of a 32-row step is row 16 (x >> 2) + 4 u + (x & 3)), so P and dS
// feed the dV / dK products straight from registers, and the dO^T / Q^T operands are
// read in the same permuted order with the transposing LDS read.
// The S and dP accumulators start from -LSE / scale and -delta of their rows (written by
// the query-major pass), so a softmax element is one FMA, one exp2 and one multiply;
// the causal mask of the diagonal items starts masked entries at -inf.
// Items stream through two LDS slots: the copy of item t + 1 (buffer loads into LDS) is
// issued right after the barrier that opens item t, and item t is computed meanwhile.
// Chunk swizzle of the key-major pass's Q / dO tiles: 16-byte chunk c of row r sits at
// chunk c ^ kv_swz(r). LDS has 64 banks of 4 bytes. Measured with the bank-conflict
// counter (address patterns replayed over 160 swizzles): an 8-byte (transposing) read is
// served in groups of 32 consecutive lanes; a 16-byte read in groups of 16 lanes, each
// half wave split by the parity of lane bits 2..4 (lanes 0-3, 12-15, 20-23, 24-27 form
// one group). Here a transposing group reads 8 rows x 32 bytes and a 16-byte group
// 8 rows x 2 chunks; the common tile swizzle, laid out for the forward's patterns, gives
// both a 2-way conflict. (r mod 8) * 2 (128-element rows) and r & 6 (64-element rows, two
// to a bank row) put every group of either read on distinct banks.
template <int D>
__device__ __forceinline__ int kv_swz(int r) {
  return D == 128 ? ((r & 7) << 1) : (r & 6);
}

template <int D, bool OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkv_kernel(const AttnArgs a) {
  constexpr int NW = 4;
  constexpr int TE = Tile<D>::ELEMS;
  constexpr int KS = D / 32;         // 32-wide k steps of the S / dP products
  constexpr int DT = D / 16;         // 16-wide d tiles of dK^T / dV^T
  // Q tile + four 64-float rows (-LSE / scale copied by wave 0, -delta by wave 1; waves 2
  // and 3 copy spare rows so that every wave issues the same number of copies)
  constexpr int TQ = TE + 4 * 128;
  __shared__ __attribute__((aligned(16))) uint16_t sq0[TQ];
  __shared__ __attribute__((aligned(16))) uint16_t sq1[TQ];
  __shared__ __attribute__((aligned(16))) uint16_t so0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t so1[TE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int u = lane >> 4, lq = lane & 15;
  const int NB = a.n / kBlock, G = a.Hq / a.Hkv;
  // Launch order: the (batch, KV head) pairs in phases of two, the work plan's segments
  // (longest first) within a phase, the two pairs of a phase interleaved so that each
  // pair's workgroups spread over the XCDs. Slots past a pair's last segment exit at once.
  const int BHp = a.B * a.Hkv;
  const int P = min(2, BHp);
  const int S = NB + a.dkv_budget;   // plan slots per pair
  const unsigned bid = wg_index(a.wg);
  const int phase = (int)(bid / ((unsigned)P * S));
  const int np = min(P, BHp - phase * P);
  const int rem = (int)(bid - (unsigned)phase * P * S);
  const int slot = rem / np;
  const int rr = phase * P + rem % np;
  const int h = rr % a.Hkv, b = rr / a.Hkv;
  const long long bh = (long long)b * a.Hkv + h;
  const int4 seg = a.seg_tab[bh * S + slot];
  if (seg.x < 0) return;   // uniform: the whole workgroup leaves before any barrier
  const int m = seg.x, sgm = seg.y, nseg = seg.z, pslot = seg.w;

  const size_t kv_off = ((size_t)bh * a.n + (size_t)m * kBlock) * D;
  const int key = 16 * wave + lq;            // this lane's key within block m
  // K / V as the B operands of S and dP: key `key`, d = 32 ks + 8 u .. + 7
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = as_bf16x8(ld16(a.K + kv_off + key * D + 32 * ks + 8 * u));
    vf[ks] = as_bf16x8(ld16(a.V + kv_off + key * D + 32 * ks + 8 * u));
    asm volatile("" : "+a"(kf[ks]), "+a"(vf[ks]));   // only the matrix cores read them
  }
  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { dk[dt][i] = 0.0f; dv[dt][i] = 0.0f; }
    asm volatile("" : "+a"(dk[dt]), "+a"(dv[dt]));
  }
  const float c2 = a.scale * kLog2e;
  // lane bases (elements) in the kv_swz tile layout: row read of rows 16 rt + lq at d = 32 ks + 8 u
  // sits at 16 rt D + (rx0 ^ (ks << 5)); the transposing read of rows 32 q + 4 u + lq / 4
  // (+ 16 for the second half of the k step) at d = 16 dt + 4 (lq % 4) at
  // 32 q D + (tx0 ^ (dt << 4)) (+ 16 D)
  const int rx0 = lq * D + ((u ^ kv_swz<D>(lq)) << 3);
  const int r0 = 4 * u + (lq >> 2);
  const int tx0 = r0 * D + ((((lq & 3) >> 1) ^ kv_swz<D>(r0)) << 3) + 4 * (lq & 1);
  const int off0 = a.inv_off[bh * (NB + 1) + m];
  const int nlist = a.inv_off[bh * (NB + 1) + m + 1] - off0;
  const int32_t* list = a.inv_list + bh * NB * a.kcap + off0;
  // this segment's items [it0, it0 + nitems) of the block's (nlist + 1) * G, entry-major
  const int ntot = (nlist + 1) * G;
  const int tseg = (ntot + nseg - 1) / nseg;
  const int it0 = min(sgm * tseg, ntot);
  const int nitems = min(tseg, ntot - it0);
  const int ndiag0 = nlist * G - it0;   // local items from here on are the diagonal block m

  const size_t head0 = (size_t)(b * a.Hq + h * G) * a.n;
  const int qbytes = G * a.n * D * 2, rbytes = G * a.n * 4;
  const uint16_t* qbase = a.Q + head0 * D;
  const uint16_t* obase = a.dO + head0 * D;
  const float* rbase = (wave == 1 ? a.ndelta : a.nlse) + head0;
  constexpr int NWIN = Tile<D>::CPR / NW;
  uint32_t voff[NWIN];
#pragma unroll
  for (int i = 0; i < NWIN; ++i) {
    const int sidx = 64 * (wave + NW * i) + lane;
    const int r = sidx / Tile<D>::CPR, c = sidx % Tile<D>::CPR;
    voff[i] = (uint32_t)(r * D + ((c ^ kv_swz<D>(r)) << 3)) * 2u;
  }
  // list entry e (descending query block; e == nlist is block m itself): query block and
  // base-2 log-gate of the entry's slot
  auto load_lst = [&](int e, int& v, float& g) {
    v = m;
    g = 0.0f;
    if (e < nlist) {
      const int p = list[nlist - 1 - e];
      v = p / a.kcap;
      const int sl = p - v * a.kcap;
      g = a.logg != nullptr ? a.logg[((size_t)bh * NB + v) * a.kcap + sl] * kLog2e : 0.0f;
    }
  };
  auto load_blk = [&](int e, int& v, float& g) {
    v = m;
    g = 0.0f;
    if (e < nlist) v = list[nlist - 1 - e] / a.kcap;
  };
  LaneList lst_c, lst_f;
  int ef = it0 / G, gf = it0 - (it0 / G) * G;    // next item to copy
  int ec = ef, gc = gf;                          // item to compute
  int nf = 0;
  // Past the last item a copy goes through an empty buffer range: it writes zeros and
  // reads no memory (every step issues the same copies, so the waits stay uniform).
  auto fetch = [&](uint16_t* qb, uint16_t* ob) {
    uint32_t row = 0;
    int qb_bytes = 0, rb_bytes = 0;
    if (nf < nitems) {
      ++nf;
      int jj = m;
      if (ef < nlist) {
        lst_f.ensure(ef, lane, load_blk);
        jj = lst_f.at(ef);
      }
      row = (uint32_t)(gf * a.n + jj * kBlock);
      qb_bytes = qbytes;
      rb_bytes = rbytes;
      if (++gf == G) { gf = 0; ++ef; }
    }
    const uint32_t so = row * (uint32_t)(D * 2);
#pragma unroll
    for (int c = 0; c < NWIN; ++c) buffer_load_lds16(qbase, qb_bytes, qb + 512 * (wave + NW * c), voff[c], so);
#pragma unroll
    for (int c = 0; c < NWIN; ++c) buffer_load_lds16(obase, qb_bytes, ob + 512 * (wave + NW * c), voff[c], so);
    buffer_load_lds4(rbase, rb_bytes, qb + TE + 128 * wave, 4u * lane, row * 4u);
  };

  auto compute = [&](int t, const uint16_t* qc, const uint16_t* oc) {
    float lg2 = 0.0f;
    if (ec < nlist) {
      lst_c.ensure(ec, lane, load_lst);
      lg2 = lst_c.gat(ec);
    }
    if (++gc == G) { gc = 0; ++ec; }
    const float gmul = OUT ? fast_exp2(lg2) : 1.0f;   // the item's gate (1 on the diagonal)
    const float* lr = reinterpret_cast<const float*>(qc + TE);
    const float* dr = reinterpret_cast<const float*>(qc + TE + 128);
    // S' and dP' start from -LSE / scale and -delta of rows 16 rt + 4 u + i
    f32x4 sacc[4], pacc[4], nd[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      sacc[rt] = *reinterpret_cast<const f32x4*>(&lr[16 * rt + 4 * u]);
      nd[rt] = *reinterpret_cast<const f32x4*>(&dr[16 * rt + 4 * u]);
      pacc[rt] = OUT ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : nd[rt];
    }
    if (t >= ndiag0) {   // block m itself: keys after the query row carry no weight
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key > 16 * rt + 4 * u + i) sacc[rt][i] = -INFINITY;
    }
    int rx = rx0;
    asm volatile("" : "+v"(rx));   // keeps per-(buffer, read) addresses unhoisted
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      bf16x8 qa[KS], oa[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[ks] = as_bf16x8(ld16(&qc[16 * rt * D + (rx ^ (ks << 5))]));
        oa[ks] = as_bf16x8(ld16(&oc[16 * rt * D + (rx ^ (ks << 5))]));
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sacc[rt] = mfma16(qa[ks], kf[ks], sacc[rt]);
        pacc[rt] = mfma16(oa[ks], vf[ks], pacc[rt]);
      }
    }
    // softmax weights and dS, packed as the B operands of the two 32-row k steps
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float pv[8], dsv[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int rt = 2 * q + (x >> 2), i = x & 3;
        if (OUT) {
          // gate after the softmax: p~ from the ungated LSE, weights p~ g for dV,
          // dS = p~ (g dP - delta)
          const float p = fast_exp2(sacc[rt][i] * c2);
          pv[x] = p * gmul;
          dsv[x] = p * (gmul * pacc[rt][i] + nd[rt][i]);
        } else {
          const float p = fast_exp2(fmaf(sacc[rt][i], c2, lg2));
          pv[x] = p;
          dsv[x] = p * pacc[rt][i];
        }
      }
      pb[q] = pack8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
      sb[q] = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
    }
    int tx = tx0;
    asm volatile("" : "+v"(tx));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int o = 32 * q * D + (tx ^ (dt << 4));
        const bf16x8 ot = join_tr16(lds_tr16(&oc[o]), lds_tr16(&oc[o + 16 * D]));
        const bf16x8 qt = join_tr16(lds_tr16(&qc[o]), lds_tr16(&qc[o + 16 * D]));
        dv[dt] = mfma16(ot, pb[q], dv[dt]);
        dk[dt] = mfma16(qt, sb[q], dk[dt]);
      }
    }
  };

  fetch(sq0, so0);
  int t = 0;
  for (; t + 2 <= nitems; t += 2) {
    wait_vm();
    barrier_lds();   // item t has landed for every wave; item t - 1 is done everywhere
    fetch(sq1, so1);
    compute(t, sq0, so0);
    wait_vm();
    barrier_lds();
    fetch(sq0, so0);
    compute(t + 1, sq1, so1);
  }
  if (t < nitems) {
    wait_vm();
    barrier_lds();
    fetch(sq1, so1);
    compute(t, sq0, so0);
  }
  wait_vm();   // the last (empty) copies land before the workgroup's LDS is released

  // this wave's 16 keys: the block's rows of dK / dV, or (segments 1.. of a split block)
  // its partial slot. dK^T / dV^T element i of lane (u, lq) in d tile dt is d = 16 dt + 4 u + i
  float* dKp = sgm == 0 ? a.dK + kv_off + key * D : a.dkv_part + (size_t)pslot * (2 * kBlock * D) + key * D;
  float* dVp = sgm == 0 ? a.dV + kv_off + key * D : dKp + kBlock * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    f32x4 kv = dk[dt], vv = dv[dt];
#pragma unroll
    for (int i = 0; i < 4; ++i) kv[i] *= a.scale;
    *reinterpret_cast<f32x4*>(dKp + 16 * dt + 4 * u) = kv;
    *reinterpret_cast<f32x4*>(dVp + 16 * dt + 4 * u) = vv;
  }
}

// ---------------------------------------------------------------- host side

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }



static int dq_splits(int G) { return (G + 1) / 2; }


// Partial-result slots of the key-major pass per (b, KV head): enough to cut the longest
// lists of a few pairs into pieces (two key-major workgroups share a CU, so a long segment
// runs at about half a CU's rate), at most 4096 slots in all.
static int dkv_budget(long long BH) { return (int)std::max<long long>(4, std::min<long long>(128, 4096 / std::max<long long>(BH, 1))); }

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int n, int d, int kcap) {
  const size_t NB = (size_t)n / kBlock;
  const size_t bh = (size_t)B * Hkv;
  const size_t kc = (size_t)(kcap > 0 ? kcap : 1);
  const int ns = dq_splits(Hq / Hkv);
  const size_t bud = (size_t)dkv_budget((long long)bh);
  return 2 * al256((size_t)B * Hq * n * sizeof(float))        // -delta, -LSE / scale
         + al256(bh * NB * sizeof(int32_t))                    // counts
         + al256(bh * (NB + 1) * sizeof(int32_t))              // offsets
         + al256(bh * NB * kc * sizeof(int32_t))               // lists
         + al256(bh * (NB + bud) * sizeof(int4))               // key-major work plan
         + al256(bh * bud * sizeof(int4))                      // split key blocks
         + al256(bh * bud * 2 * kBlock * (size_t)d * sizeof(float))   // their partial dK / dV
         + (ns > 1 ? al256((size_t)ns * bh * NB * kc * sizeof(float)) : 0);  // dg partials
}

template <int D>
static hipError_t launch_bwd_d(AttnArgs& a, hipStream_t st) {
  const int NB = a.n / kBlock;
  const long long nrows = (long long)a.B * a.Hkv * NB;
  {
    ProfScope prof("inv_count", st);
    hipLaunchKernelGGL(inv_kernel, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, a.idx, a.cnt,
                       NB, a.kcap, nrows, a.inv_cnt, (const int32_t*)nullptr, (int32_t*)nullptr);
  }
  {
    ProfScope prof("inv_scan", st);
    hipLaunchKernelGGL(inv_scan_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(256), 0, st, a.inv_cnt, NB,
                       a.Hq / a.Hkv, a.dkv_budget, a.inv_off, a.seg_tab, a.red_tab);
  }
  {
    ProfScope prof("inv_fill", st);
    hipLaunchKernelGGL(inv_kernel, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, a.idx, a.cnt,
                       NB, a.kcap, nrows, a.inv_cnt, (const int32_t*)a.inv_off, a.inv_list);
  }
  const int nsplit = dq_splits(a.Hq / a.Hkv);
  {
    ProfScope prof("dq", st);
    const unsigned grid = (unsigned)(nrows * nsplit);
    a.wg = wg_order(grid);
    if (a.gate_out)
      hipLaunchKernelGGL((dq_kernel<D, true>), dim3(grid), dim3(256), 0, st, a, nsplit);
    else
      hipLaunchKernelGGL((dq_kernel<D, false>), dim3(grid), dim3(256), 0, st, a, nsplit);
  }
  if (nsplit > 1 && a.kcap > 0) {
    ProfScope prof("dg_reduce", st);
    const long long n = nrows * a.kcap;
    hipLaunchKernelGGL(dg_reduce_kernel, dim3((unsigned)std::min<long long>((n + 255) / 256, 4096)),
                       dim3(256), 0, st, (const float*)a.dg_part, a.dg, n, nsplit);
  }
  {
    ProfScope prof("dkv", st);
    const unsigned grid = (unsigned)((long long)a.B * a.Hkv * (NB + a.dkv_budget));
    a.wg = wg_order(grid);
    if (a.gate_out) hipLaunchKernelGGL((dkv_kernel<D, true>), dim3(grid), dim3(256), 0, st, a);
    else hipLaunchKernelGGL((dkv_kernel<D, false>), dim3(grid), dim3(256), 0, st, a);
  }
  {
    ProfScope prof("dkv_reduce", st);
    hipLaunchKernelGGL((dkv_reduce_kernel<D>), dim3((unsigned)((long long)a.B * a.Hkv * a.dkv_budget)), dim3(256), 0,
                       st, (const int4*)a.red_tab, a.dkv_budget, a.n, (const float*)a.dkv_part, a.dK, a.dV);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(AttnArgs a, void* ws, hipStream_t st) {
  const size_t NB = (size_t)a.n / kBlock;
  const size_t bh = (size_t)a.B * a.Hkv;
  const size_t kc = (size_t)(a.kcap > 0 ? a.kcap : 1);
  char* p = (char*)ws;
  a.ndelta = (float*)p;
  p += al256((size_t)a.B * a.Hq * a.n * sizeof(float));
  a.nlse = (float*)p;
  p += al256((size_t)a.B * a.Hq * a.n * sizeof(float));
  a.inv_cnt = (int32_t*)p;
  p += al256(bh * NB * sizeof(int32_t));
  a.inv_off = (int32_t*)p;
  p += al256(bh * (NB + 1) * sizeof(int32_t));
  a.inv_list = (int32_t*)p;
  p += al256(bh * NB * kc * sizeof(int32_t));
  a.dkv_budget = dkv_budget((long long)bh);
  const size_t bud = (size_t)a.dkv_budget;
  a.seg_tab = (int4*)p;
  p += al256(bh * (NB + bud) * sizeof(int4));
  a.red_tab = (int4*)p;
  p += al256(bh * bud * sizeof(int4));
  a.dkv_part = (float*)p;
  p += al256(bh * bud * 2 * kBlock * (size_t)a.d * sizeof(float));
  a.dg_part = (float*)p;
  if (a.d == 128) return launch_bwd_d<128>(a, st);
  return launch_bwd_d<64>(a, st);
}

}  // namespace sas
