// Decode step in the inference form of SAS ([SAS-ja] "仕組み", Algorithm 2 / section 5.1):
// the new token of each sequence attends, without gates, to its current block plus the
// Top-K history blocks picked from s. Per (sequence, KV head) the G query heads share the
// selected K/V blocks, so each block is read from HBM once for all G heads.
//
// The work is HBM-bound: the kernel's job is to keep enough bytes in flight. The block list
// of each (sequence, KV head) is split into chunks so the launch fills the chip; each chunk
// is one single-wave workgroup that streams its K/V blocks, in 32-key halves, through a
// ring of LDS buffer sets (buffer loads into LDS, swizzled tiles; rows past the cache end
// read as zero) and computes, like the prefill forward, S^T = K Q^T and O^T += V^T P^T with
// 32x32x16 bf16 MFMAs, the G query heads forming the query columns (columns G..31 are
// zero). The chunk's block list is held one entry per lane, so no step waits on an index
// load. A wave needs no barrier: it waits only for its own copies. With one chunk per
// (sequence, KV head) the output is written directly; otherwise each chunk writes a
// partial (running max, running sum, unnormalised output) per query head and a second
// kernel merges the partials with log-sum-exp rescaling.
#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

constexpr float kDecRescaleThreshold = 8.0f;   // log2 of the largest unnormalised exponential

// The same copy from a base address and range that are equal in every lane but that the
// compiler cannot prove uniform (a page's address, computed from a page id read out of a
// lane-held list): both are moved to scalar registers first. Otherwise the compiler wraps
// each copy in a loop over the distinct resources of the wave's lanes (four
// v_readfirstlane, two compares and an exec-mask loop per copy), which stalls the issue of
// the copies behind it.
__device__ __forceinline__ void buffer_load_lds16_u(const void* base, int bytes, void* lds, uint32_t voffset) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  buffer_load_lds16(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes),
                    lds, voffset, 0u);
}

// 32-key half blocks through a ring of 4 LDS buffer sets: half block u+3 is copied in
// while u is computed, so about three half blocks (48 KB) are in flight per wave.
//
// PAGED: the cache is a pool of 64-token pages and a page table per sequence. The list
// then holds page ids, and every half block is copied through a buffer resource that
// starts at its page and covers only its valid rows, so rows past kv_len (which a page
// allocator leaves unwritten) read as zero rather than whatever the page holds.
//
// EARLY: the mass-threshold early stop ([S2O-ja] "S2O: オンライン置換によるスパースアテンション
// の早期停止", section "2. 早期停止ルール"): the list (one chunk, at most 64 entries) is
// sorted in the wave by descending order key after the current block; per query head the
// softmax mass a block adds is compared with the mass accumulated before it, the block is
// kept and, once the ratio falls below tau, that head takes no further block. The wave
// stops copying when every head has stopped.
//
// SEL: the block selection in the same launch (sas_decode_topk, and with PAGED
// sas_decode_paged_topk). The wave loads its row of history scores, issues the copies of
// its current block (they depend on kv_len, and paged on its page, only), then finds the
// row's Top-K exactly as the selection kernel does (topk_cut / topk_walk, decode mode: the
// valid scores are the row's first (kv_len - 1) / 64) while those copies are in flight,
// and keeps the kept block indices, ascending, in LDS for the block list. SEL = 1 ranks
// the row's score columns (column m is block m); SEL = 2 ranks candidate slots, each a
// (score, block) pair with empty slots marked by block -1, the slots in ascending block
// order (so a tie still goes to the lower block), as the candidates kernel writes them.
template <int D, bool PAGED, bool EARLY, int SEL>
__global__ __launch_bounds__(64) void decode_split_kernel(const DecodeArgs a) {
  constexpr int HE = 32 * D;   // elements of a 32-row half tile
  __shared__ __attribute__((aligned(16))) uint16_t sk0[HE];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[HE];
  __shared__ __attribute__((aligned(16))) uint16_t sk2[HE];
  __shared__ __attribute__((aligned(16))) uint16_t sk3[HE];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[HE];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[HE];
  __shared__ __attribute__((aligned(16))) uint16_t sv2[HE];
  __shared__ __attribute__((aligned(16))) uint16_t sv3[HE];
  __shared__ int s_sel[SEL ? kDecSelMax + 1 : 1];   // (SEL) the kept blocks, ascending; a spare slot
  const int lane = threadIdx.x;
  const int hl = lane >> 5, ql = lane & 31;
  const int G = a.Hq / a.Hkv;
  const unsigned bid = wg_index(a.wg);
  const int chunk = bid % a.nchunk;
  const long long bh = bid / a.nchunk;
  const int h = (int)(bh % a.Hkv), b = (int)(bh / a.Hkv);
  const int t0 = chunk * a.bpc;
  const int32_t* idx_row = a.idx + bh * a.kcap;
  const float* lg_row = a.logg != nullptr ? a.logg + bh * a.kcap : nullptr;
  // The raw entries of the chunk's first list window (lane i: position t0 + i) depend on
  // neither kv_len nor cnt: loaded together with them, the first copies need one memory
  // latency less. Which of them count is decided once cnt and kv_len are in. (Not in the
  // early-stop form: its in-wave sort leaves no registers for them, and the compiler
  // then moves state to scratch memory, which costs far more than the latency.)
  int pre_v = 0;
  float pre_g = 0.0f;
  if (!EARLY && !SEL && t0 + lane > 0 && t0 + lane <= a.kcap) {
    pre_v = idx_row[t0 + lane - 1];
    if (lg_row != nullptr) pre_g = lg_row[t0 + lane - 1];
  }
  // (SEL) The row's scores likewise: every column a sequence of this cache can have as
  // history ((Lmax - 1) / 64, at most kDecSelMaxCols, and the row holds s_ld >= that many),
  // so the loads need not wait for kv_len; the columns past the sequence's own history are
  // masked once it is known.
  // (SEL = 2: the row's candidate slots, s_ld of them, and their blocks.)
  constexpr int PL = SEL ? kDecSelMaxCols / 64 : 1;
  float x[PL];
  int xid[SEL == 2 ? PL : 1];
  int ncol = 0;
  if constexpr (SEL) {
    ncol = SEL == 2 ? a.s_ld : min(a.s_ld, (int)((a.Lmax - 1) / kBlock));
    const int nld = (ncol + 63) >> 6;
    const float* srow = a.s + bh * a.s_ld;
#pragma unroll
    for (int i = 0; i < PL; ++i) x[i] = i < nld ? srow[min(lane + 64 * i, ncol - 1)] : -INFINITY;
    if constexpr (SEL == 2) {
      const int32_t* irow = a.s_id + bh * a.s_ld;
#pragma unroll
      for (int i = 0; i < PL; ++i) xid[i] = i < nld ? irow[min(lane + 64 * i, ncol - 1)] : -1;
    }
  }
  const int L = min(max(a.kv_len[b], 1), (int)a.Lmax);
  const int cur = (L - 1) / kBlock;
  const uint16_t* Kh = a.Kc + (size_t)bh * a.Lmax * D;
  const uint16_t* Vh = a.Vc + (size_t)bh * a.Lmax * D;
  // The copies' byte range is the sequence's own tokens: cache rows at or past kv_len (in
  // the current block) read as zero, whatever the cache holds there. Their keys are masked
  // anyway, but a weight of zero times a NaN value row would still be NaN.
  // (L * D * 2 <= Lmax * D * 2, checked on the host to fit 31 bits.)
  const int cbytes = L * D * 2;
  constexpr int NWIN = Tile<D>::CPR / 2;   // 1 KB windows per half tile (one wave copies all)
  uint32_t voff[NWIN];
#pragma unroll
  for (int i = 0; i < NWIN; ++i) {
    const int sidx = 64 * i + lane;
    const int rr = sidx / Tile<D>::CPR, c = sidx % Tile<D>::CPR;
    voff[i] = (uint32_t)(rr * D + ((c ^ Tile<D>::swz(rr)) << 3)) * 2u;
  }
  // the G query heads as the B operand of S^T = K Q^T: lane holds query column ql,
  // d = 16 ks + 8 hl + e; columns ql >= G are zero (loaded before the selection, whose
  // wavefront fences would keep them behind it)
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = ql < G ? as_bf16x8(ld16(a.q + ((size_t)b * a.Hq + h * G + ql) * D + 16 * ks + 8 * hl)) : bf16x8{};

  int cnt = 0;
  bool early_cur = false;   // (SEL) the current block's copies were issued before the selection
  if constexpr (SEL) {
    // positions ranked: the history columns (SEL = 1; cur <= ncol) or every candidate slot
    const int valid = SEL == 2 ? ncol : cur;
    const int k = min(a.topk, cur);   // (SEL = 2: at least min(K, cur) slots hold blocks)
    const int nreg = __builtin_amdgcn_readfirstlane((valid + 63) >> 6);
    // The scores (and q) are awaited before the current block's copies are issued: the
    // memory counter drains in issue order, so a wait for them after the copies would be a
    // wait for the copies too, and the search would start only once those had landed.
    wait_vm();
    uint32_t key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      float v = -INFINITY;
      if (i < nreg) v = x[i];
      bool in = lane + 64 * i < valid;
      if constexpr (SEL == 2) in = in && xid[i] >= 0 && xid[i] < cur;   // an empty slot is no block
      v = (in && v == v) ? v : -INFINITY;   // NaN ranks as -inf
      v = v == 0.0f ? 0.0f : v;             // -0 -> +0
      key[i] = in ? order_key(v) : 0u;
    }
    if (t0 == 0) {
      // the current block's two halves into the first two ring slots, in flight during
      // the search (paged: its page, rows at or past kv_len read as zero; a page id out of
      // range reads nothing)
      int pg = 0;
      if constexpr (PAGED) {
        pg = a.page_table[(size_t)b * a.max_pages + cur];
        if (pg < 0 || pg >= a.num_pages) pg = -1;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        uint16_t* kb = u == 0 ? sk0 : sk1;
        uint16_t* vb = u == 0 ? sv0 : sv1;
        if constexpr (PAGED) {
          const size_t off = ((size_t)max(pg, 0) * a.Hkv + h) * (size_t)(kBlock * D) + (size_t)(32 * u) * D;
          const int pbytes = pg < 0 ? 0 : min(max(L - cur * kBlock - 32 * u, 0), 32) * D * 2;
#pragma unroll
          for (int i = 0; i < NWIN; ++i) buffer_load_lds16_u(a.Kc + off, pbytes, kb + 512 * i, voff[i]);
#pragma unroll
          for (int i = 0; i < NWIN; ++i) buffer_load_lds16_u(a.Vc + off, pbytes, vb + 512 * i, voff[i]);
        } else {
          const uint32_t so = ((uint32_t)cur * kBlock + 32u * u) * (uint32_t)(D * 2);
#pragma unroll
          for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Kh, cbytes, kb + 512 * i, voff[i], so);
#pragma unroll
          for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Vh, cbytes, vb + 512 * i, voff[i], so);
        }
      }
      early_cur = true;
    }
    if (k > 0) {
      uint32_t T;
      int need_eq;
      topk_cut<PL, true>(key, nreg, valid, k, T, need_eq);   // the wave has its SIMD to itself
      if (need_eq == 0) {   // no tie at the cut: every lane writes, the unkept ones to a spare slot
        auto put = [&](int i, int pos, bool kept) {
          s_sel[kept ? pos : kDecSelMax] = SEL == 2 ? xid[i] : lane + 64 * i;
        };
        if (nreg <= PL / 2) topk_walk_gt<PL / 2>(key, T, put);
        else topk_walk_gt<PL>(key, T, put);
      } else {
        topk_walk(key, nreg, T, need_eq, [&](int i, int pos) { s_sel[pos] = SEL == 2 ? xid[i] : lane + 64 * i; });
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");   // the list, for every lane
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cnt = max(k, 0);
    if (a.idx_out != nullptr && chunk == 0) {
      for (int p = lane; p < a.kcap; p += 64) a.idx_out[bh * a.kcap + p] = p < cnt ? s_sel[p] : -1;
      if (lane == 0) a.cnt_out[bh] = cnt;
    }
  } else {
    cnt = min(max(a.cnt[bh], 0), min(a.kcap, cur));
  }
  // list position t: 0 is the current block, t >= 1 the selected block idx[t - 1]
  // (a chunk past the end of a short list is empty: t1 == t0)
  const int t1 = max(t0, min(t0 + a.bpc, cnt + 1));

  // The chunk's list positions, one per lane (lane i: position t0 + i): block and base-2
  // log-gate; an ignored entry reads block 0 with weight 0.
  LaneList lst;
  auto load_lst = [&](int i, int& v, float& g) {
    const int t = t0 + i;
    v = cur;
    g = 0.0f;
    if (t > 0 && t < t1) {
      if (SEL) {   // the list selected above (at most kDecSelMax entries: one window)
        v = s_sel[t - 1];
        g = 0.0f;
      } else if (!EARLY && i < 64) {   // the first window, loaded at the start
        v = pre_v;
        g = pre_g * kLog2e;
      } else {
        v = idx_row[t - 1];
        g = lg_row != nullptr ? lg_row[t - 1] * kLog2e : 0.0f;
      }
      if (v < 0 || v >= cur) { v = 0; g = -INFINITY; }
    }
    if (PAGED) {   // logical block -> page; a page id out of range reads nothing
      const int pg = a.page_table[(size_t)b * a.max_pages + v];
      v = pg;
      if (pg < 0 || pg >= a.num_pages) { v = -1; g = -INFINITY; }
    }
    if (EARLY) {
      // bitonic sort of the 64 entries by (order key descending, block ascending); the
      // current block (position 0) first, unused positions last
      float key = t == 0 ? INFINITY : -INFINITY;
      int ord = t == 0 ? -1 : 0x7FFFFFFF;
      if (t > 0 && t < t1) {
        key = a.order[bh * a.kcap + t - 1];
        if (key != key) key = -INFINITY;
        ord = v;
      }
      for (int kk = 2; kk <= 64; kk <<= 1)
        for (int j = kk >> 1; j > 0; j >>= 1) {
          const float pk = __shfl_xor(key, j, 64);
          const int po = __shfl_xor(ord, j, 64), pv = __shfl_xor(v, j, 64);
          const float pg = __shfl_xor(g, j, 64);
          const bool mine_first = key > pk || (key == pk && ord < po);
          const bool want_first = ((lane & j) == 0) == ((lane & kk) == 0);
          if (mine_first != want_first && !(key == pk && ord == po)) { key = pk; ord = po; v = pv; g = pg; }
        }
    }
  };
  LaneList lstf;   // the same list for the copies, which run ahead
  const int nhalf = 2 * (t1 - t0);
  int uf = 0;   // next half block to copy (stays at nhalf - 1 once reached)
  // valid keys of half block u of this chunk: all 32, except in the current block
  auto half_keys = [&](int u) {
    return t0 + (u >> 1) == 0 ? min(max(L - cur * kBlock - 32 * (u & 1), 0), 32) : 32;
  };
  auto fetch = [&](uint16_t* kb, uint16_t* vb) {
    const int uu = max(min(uf, nhalf - 1), 0);
    lstf.ensure(uu >> 1, lane, load_lst);
    const int m = lstf.at(uu >> 1);
    if (PAGED) {
      const size_t off = ((size_t)max(m, 0) * a.Hkv + h) * (size_t)(kBlock * D) + (size_t)(32 * (uu & 1)) * D;
      const int bytes = m < 0 ? 0 : half_keys(uu) * D * 2;
#pragma unroll
      for (int i = 0; i < NWIN; ++i) buffer_load_lds16_u(a.Kc + off, bytes, kb + 512 * i, voff[i]);
#pragma unroll
      for (int i = 0; i < NWIN; ++i) buffer_load_lds16_u(a.Vc + off, bytes, vb + 512 * i, voff[i]);
    } else {
      const uint32_t so = ((uint32_t)m * kBlock + 32u * (uu & 1)) * (uint32_t)(D * 2);
#pragma unroll
      for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Kh, cbytes, kb + 512 * i, voff[i], so);
#pragma unroll
      for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Vh, cbytes, vb + 512 * i, voff[i], so);
    }
    ++uf;
  };
  constexpr int PER = 2 * NWIN;   // copies per half block
  static_assert(2 * PER < 64, "copies in flight exceed the vmcnt range");

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.0f;
  float mref = -INFINITY, lrow = 0.0f;
  const float c2 = a.scale * kLog2e;
  const int g16 = lane >> 4, lp = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (lp >> 2), tr_d = 16 * (g16 & 1) + 4 * (lp & 3);
  const int rx0 = ql * D + ((hl ^ Tile<D>::swz(ql)) << 3);
  const int tx0 = tr_row * D + ((((tr_d >> 3) ^ Tile<D>::swz(tr_row))) << 3) + (tr_d & 7);

  // early stop state per query column: stopped, history blocks taken, the block's mass
  // so far (this lane's rows) and the column's mass before the block (same frame)
  bool done = !EARLY || ql >= G;
  int used = 0;
  float dlb = 0.0f, lbefore = 0.0f;
  int uc = 0;   // half block being computed
  auto step = [&](const uint16_t* kc, const uint16_t* vc, uint16_t* kn, uint16_t* vn) {
    wait_vm_n<2 * PER>();   // this half block has landed; the next two may still be in flight
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of the buffer about to be refilled are done
    const int u = uc++;
    lst.ensure(u >> 1, lane, load_lst);
    const int m = lst.at(u >> 1);
    const float lg2 = lst.gat(u >> 1);
    fetch(kn, vn);
    int rx = rx0, tx = tx0;
    asm volatile("" : "+v"(rx), "+v"(tx));
    f32x16 st = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) st = mfma32(as_bf16x8(ld16(&kc[rx ^ (ks << 4)])), qf[ks], st);
    bf16x8 va[D / 32][2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r0 = 16 * hh;
        va[dt][hh] = join_tr16(lds_tr16(&vc[r0 * D + (tx ^ ((4 * dt) << 3))]),
                               lds_tr16(&vc[(r0 + 8) * D + (tx ^ ((4 * dt ^ 2) << 3))]));
      }
    // keys past the end of the cache (only in the current block) do not count
    if (PAGED) {
      const int lim = half_keys(u);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hl + (i & 3);
        if (key >= lim) st[i] = -INFINITY;
      }
    } else {
      const int key0 = m * kBlock + 32 * (u & 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 8 * (i >> 2) + 4 * hl + (i & 3);
        if (key0 + key >= L) st[i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[i]);
    mx = half_max(mx);
    const float bmax = mx * c2 + lg2;
    const bool hist_block = EARLY && (t0 + (u >> 1)) > 0;
    if (hist_block && (u & 1) == 0) {   // a history block starts
      dlb = 0.0f;
      lbefore = half_sum(lrow);
    }
    if (__any(bmax > mref + kDecRescaleThreshold)) {
      const float mnew = fmaxf(mref, bmax);
      const float alpha = mnew == -INFINITY ? 1.0f : fast_exp2(mref - mnew);
      mref = mnew;
      lrow *= alpha;
      if (EARLY) { dlb *= alpha; lbefore *= alpha; }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
    // a column whose reference is still -inf has seen only masked keys: weight 0; a
    // stopped column takes no further block
    const bool skip = EARLY && hist_block && done;
    const float off = (mref == -INFINITY || skip) ? -INFINITY : lg2 - mref;
    float ls = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(st[i] * c2 + off);
      st[i] = p;
      ls += p;
    }
    lrow += ls;
    if (hist_block) {
      dlb += ls;
      if (u & 1) {   // the block is complete: keep it, and stop once its mass is small
        const float dl = half_sum(dlb);
        if (!done) {
          ++used;
          if (dl < a.tau * lbefore) done = true;
        }
      }
    }
    bf16x8 pf[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int o = 8 * hh;
      pf[hh] = pack8(st[o], st[o + 1], st[o + 2], st[o + 3], st[o + 4], st[o + 5], st[o + 6], st[o + 7]);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) oacc[dt] = mfma32(va[dt][hh], pf[hh], oacc[dt]);
  };
  // whole rounds of 4 half blocks without conditions inside, then the remainder
  if (early_cur) {
    uf = 2;   // (SEL) the current block's halves are already on their way
  } else {
    fetch(sk0, sv0);
    fetch(sk1, sv1);
  }
  fetch(sk2, sv2);
  const int nfull = nhalf & ~3;
  bool stopped = false;
  for (int it = 0; it < nfull; it += 4) {
    step(sk0, sv0, sk3, sv3);
    step(sk1, sv1, sk0, sv0);
    step(sk2, sv2, sk1, sv1);
    step(sk3, sv3, sk2, sv2);
    if (EARLY && __all(done)) { stopped = true; break; }   // every head has stopped
  }
  if (!stopped) {
    if (nfull < nhalf) step(sk0, sv0, sk3, sv3);
    if (nfull + 1 < nhalf) step(sk1, sv1, sk0, sv0);
    if (nfull + 2 < nhalf) step(sk2, sv2, sk1, sv1);
  }
  wait_vm();
  if (EARLY && a.used != nullptr && hl == 0 && ql < G) a.used[(size_t)b * a.Hq + h * G + ql] = used;

  const float l = half_sum(lrow);
  if (a.nchunk == 1) {
    // the whole list in one chunk: write the normalised output directly
    if (ql < G) {
      const float inv = 1.0f / l;
      uint16_t* o = a.o + ((size_t)b * a.Hq + h * G + ql) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = 32 * dt + 8 * g4 + 4 * hl;
          bf16x4 v;
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = (__bf16)(oacc[dt][4 * g4 + x] * inv);
          *reinterpret_cast<bf16x4*>(o + d0) = v;
        }
    }
    return;
  }
  // partial of this chunk for query head ql < G: (m, l, unnormalised o)
  if (ql < G) {
    float* out = a.part + (((size_t)bh * a.nchunk + chunk) * G + ql) * (D + 2);
    if (hl == 0) { out[0] = mref; out[1] = l; }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dt + 8 * g4 + 4 * hl;
#pragma unroll
        for (int x = 0; x < 4; ++x) out[2 + d0 + x] = oacc[dt][4 * g4 + x];
      }
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const DecodeArgs a) {
  const int G = a.Hq / a.Hkv;
  const long long bq = blockIdx.x;                 // b * Hq + hq
  const int hq = (int)(bq % a.Hq), b = (int)(bq / a.Hq);
  const int h = hq / G, g = hq % G;
  const long long bh = (long long)b * a.Hkv + h;
  const float* base = a.part + (size_t)bh * a.nchunk * G * (D + 2);
  const int dd = threadIdx.x;
  float M = -INFINITY;
  for (int c = 0; c < a.nchunk; ++c) M = fmaxf(M, base[((size_t)c * G + g) * (D + 2)]);
  float o = 0.0f, l = 0.0f;
  for (int c = 0; c < a.nchunk; ++c) {
    const float* p = base + ((size_t)c * G + g) * (D + 2);
    if (p[0] == -INFINITY) continue;
    const float sc = exp2f(p[0] - M);
    o += sc * p[2 + dd];
    l += sc * p[1];
  }
  a.o[bq * D + dd] = f2bf(o / l);
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int d, int kcap) {
  // Upper bound over every chunking the launcher may pick (one block per chunk).
  const size_t G = (size_t)Hq / Hkv;
  return (size_t)B * Hkv * (size_t)(kcap + 1) * G * (d + 2) * sizeof(float);
}

constexpr long long kDecTargetWG = 512;   // aim for about this many single-wave workgroups

// Chunking of the block lists: enough chunks for about kDecTargetWG workgroups, at least 2
// blocks per chunk; the early stop walks one sorted list per head (one chunk).
void decode_plan(DecodeArgs& a) {
  const long long pairs = (long long)a.B * a.Hkv;
  const int nblk = a.kcap + 1;
  int chunks = (int)((kDecTargetWG + pairs - 1) / pairs);
  chunks = max(1, min(chunks, (nblk + 1) / 2));
  if (a.order != nullptr) chunks = 1;
  a.bpc = (nblk + chunks - 1) / chunks;
  a.nchunk = (nblk + a.bpc - 1) / a.bpc;
}

size_t decode_part_bytes(const DecodeArgs& a) {
  if (a.nchunk <= 1) return 0;
  const size_t G = (size_t)a.Hq / a.Hkv;
  return (size_t)a.B * a.Hkv * (size_t)a.nchunk * G * (a.d + 2) * sizeof(float);
}

hipError_t launch_decode(DecodeArgs a, hipStream_t st) {
  const long long pairs = (long long)a.B * a.Hkv;
  decode_plan(a);
  const unsigned grid = (unsigned)(pairs * a.nchunk);
  a.wg = wg_order(grid);
  {
    const bool paged = a.page_table != nullptr, early = a.order != nullptr, sel = a.s != nullptr;
    ProfScope prof(early ? "decode_early_stop"
                   : paged ? (sel ? (a.s_id != nullptr ? "decode_paged_candidates_topk" : "decode_paged_topk")
                                  : "decode_paged")
                   : sel ? (a.s_id != nullptr ? "decode_candidates_topk" : "decode_topk") : "decode", st);
    if (a.d == 128) {
      if (early) hipLaunchKernelGGL((decode_split_kernel<128, false, true, 0>), dim3(grid), dim3(64), 0, st, a);
      else if (paged && sel && a.s_id != nullptr) hipLaunchKernelGGL((decode_split_kernel<128, true, false, 2>), dim3(grid), dim3(64), 0, st, a);
      else if (paged && sel) hipLaunchKernelGGL((decode_split_kernel<128, true, false, 1>), dim3(grid), dim3(64), 0, st, a);
      else if (paged) hipLaunchKernelGGL((decode_split_kernel<128, true, false, 0>), dim3(grid), dim3(64), 0, st, a);
      else if (sel && a.s_id != nullptr) hipLaunchKernelGGL((decode_split_kernel<128, false, false, 2>), dim3(grid), dim3(64), 0, st, a);
      else if (sel) hipLaunchKernelGGL((decode_split_kernel<128, false, false, 1>), dim3(grid), dim3(64), 0, st, a);
      else hipLaunchKernelGGL((decode_split_kernel<128, false, false, 0>), dim3(grid), dim3(64), 0, st, a);
    } else {
      if (early) hipLaunchKernelGGL((decode_split_kernel<64, false, true, 0>), dim3(grid), dim3(64), 0, st, a);
      else if (paged && sel && a.s_id != nullptr) hipLaunchKernelGGL((decode_split_kernel<64, true, false, 2>), dim3(grid), dim3(64), 0, st, a);
      else if (paged && sel) hipLaunchKernelGGL((decode_split_kernel<64, true, false, 1>), dim3(grid), dim3(64), 0, st, a);
      else if (paged) hipLaunchKernelGGL((decode_split_kernel<64, true, false, 0>), dim3(grid), dim3(64), 0, st, a);
      else if (sel && a.s_id != nullptr) hipLaunchKernelGGL((decode_split_kernel<64, false, false, 2>), dim3(grid), dim3(64), 0, st, a);
      else if (sel) hipLaunchKernelGGL((decode_split_kernel<64, false, false, 1>), dim3(grid), dim3(64), 0, st, a);
      else hipLaunchKernelGGL((decode_split_kernel<64, false, false, 0>), dim3(grid), dim3(64), 0, st, a);
    }
  }
  if (a.nchunk > 1) {
    ProfScope prof("decode_merge", st);
    if (a.d == 128)
      hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)(a.B * a.Hq)), dim3(128), 0, st, a);
    else
      hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sas
