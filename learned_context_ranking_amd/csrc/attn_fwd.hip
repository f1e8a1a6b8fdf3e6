// Log-gated block-sparse attention forward on bf16 MFMA (gfx950).
//
// [SAS-ja] "仕組み", eq. (9) / [SAS-ko] "어떻게 동작하나": for query block j,
//   o = softmax(scale * q K_S^T + log g_S) V_S,  S = B_j (causal, gate 1) U the selected blocks,
// with log g of a selected block added to every logit of its 64 tokens. The gate add and
// the causal mask are fused into the logit tile; no attention matrix leaves registers.
//
// Work item: one workgroup per (batch, KV head, query block j, head split). The workgroup
// serves HPW query heads of the KV group; each head's 64 rows are owned by 64/ROWS waves,
// so one staged K/V block feeds HPW * 64 query rows (GQA reuse).
//
// Orientation: each wave computes S^T = K Q^T (keys x queries) with 32x32x16 MFMAs. A lane
// then holds one query column and 32 of its 64 keys: the row softmax needs one cross-lane
// exchange (lane ^ 32), and the probabilities are already laid out as the B operand of
// O^T += V^T P^T. V stays in its natural row-major layout in LDS and the V^T operand is
// read with the transposing ds_read_b64_tr_b16, in the key order the accumulator uses.
//
// Two kernels share this structure: fwd3_kernel (d = 128, two or more query heads per KV
// head; three waves per SIMD, see its comment) and fwd_kernel (the other shapes).
//
// Pipeline of fwd_kernel: the next block's K/V tiles are copied from global memory straight
// into the other LDS buffer (buffer loads into LDS with a scalar per-block offset, swizzled tiles)
// while the current block is computed; one barrier per block. The copy is issued on every
// step (past the end of the list it repeats the last block) and the steps run in whole
// rounds of two, so the compiler's tracking of the copies in flight stays exact and it
// never waits for the copy of the next block before reading the current one. Waves of a
// missing head (odd G in the last split) take part in the copies and barriers only. Blocks are visited current block first, so every row's reference maximum is
// finite from the start (each query sees itself). The reference maximum is only moved when
// a row's maximum grows by more than 2^8 (exponentials stay <= 256), which skips nearly
// all rescales of the output accumulator.
#include <type_traits>

#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

constexpr float kRescaleThreshold = 8.0f;   // log2 of the largest unnormalised exponential

// 32 rows per wave (NTILE 1) is sized to leave room for two waves per SIMD.
template <int D, int NTILE, int NW, bool OUT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NTILE == 1 ? 2 : 1, NTILE == 1 ? 2 : 1)))
void fwd_kernel(const AttnArgs a, int nsplit, int hpw) {
  constexpr int NT = 64 * NW;              // threads
  constexpr int WPH = 2 / NTILE;           // waves per query head (64 rows / (32 * NTILE))
  // Two K/V buffers as distinct LDS objects, always selected at compile time: the compiler
  // can then prove that the asynchronous copy into one buffer does not alias reads of the
  // other and does not wait for the copy before computing.
  __shared__ __attribute__((aligned(16))) uint16_t sk0[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sv0[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sv1[Tile<D>::ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int hl = lane >> 5, ql = lane & 31;
  const int NB = a.n / kBlock, G = a.Hq / a.Hkv;

  // Heaviest query blocks first; consecutive workgroups differ in (batch, head), so a KV head
  // and all its query-head splits stay on one XCD (one L2) when B * Hkv is a multiple of 8.
  const int BH = a.B * a.Hkv;
  const int per_j = BH * nsplit;
  const unsigned bid = wg_index(a.wg);
  const int j = NB - 1 - (int)(bid / per_j);
  const int r = bid % per_j;
  const int split = r / BH;             // splits of one (b, h) are BH workgroups apart: same XCD when BH % 8 == 0
  const int h = (r % BH) % a.Hkv, b = (r % BH) / a.Hkv;
  const int head0 = split * hpw;
  const int nheads = min(hpw, G - head0);
  const int whead = wave / WPH;            // head of this wave within the split
  const int wrow0 = (wave % WPH) * 32 * NTILE;
  const bool active = whead < nheads;
  const int hq = h * G + head0 + (active ? whead : 0);

  const size_t kv_off = ((size_t)(b * a.Hkv + h) * a.n) * D;
  const uint16_t* Kh = a.K + kv_off;
  const uint16_t* Vh = a.V + kv_off;
  const size_t q_off = ((size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock + wrow0) * D;
  const size_t sel_row = (size_t)(b * a.Hkv + h) * NB + j;
  const int cnt_j = min(max(a.cnt[sel_row], 0), min(a.kcap, j));
  const int32_t* idx_row = a.idx + sel_row * a.kcap;
  const float* lg_row = a.logg != nullptr ? a.logg + sel_row * a.kcap : nullptr;

  // Q as the B operand of S^T = K Q^T: lane holds query 32*nt + l%32, d = 16*ks + 8*(l/32) + e.
  bf16x8 qf[NTILE][D / 16];
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[nt][ks] = as_bf16x8(ld16(a.Q + q_off + (32 * nt + ql) * D + 16 * ks + 8 * hl));

  // Block t of the visit order: t = 0 is block j itself, t >= 1 the selected block
  // idx[t - 1] (an ignored entry stages block 0 with weight 0). The selection row is held
  // one entry per lane. tc: block being computed; tf: next block to copy (stays at cnt_j).
  auto load_sel = [&](int i, int& v, float& g) {
    v = i < cnt_j ? idx_row[i] : 0;
    g = (i < cnt_j && lg_row != nullptr) ? lg_row[i] * kLog2e : 0.0f;
  };
  LaneList sel_c, sel_f;
  int tc = 0, tf = 0;
  constexpr int NWIN = Tile<D>::CPR / NW;
  static_assert(Tile<D>::CPR % NW == 0, "tile windows must split evenly over the waves");
  uint32_t voff[NWIN];
#pragma unroll
  for (int i = 0; i < NWIN; ++i) {
    const int sidx = 64 * (wave + NW * i) + lane;
    const int rr = sidx / Tile<D>::CPR, c = sidx % Tile<D>::CPR;
    voff[i] = (uint32_t)(rr * D + ((c ^ Tile<D>::swz(rr)) << 3)) * 2u;
  }
  const int kvbytes = a.n * D * 2;
  auto fetch = [&](uint16_t* kb, uint16_t* vb) {
    int mb = j;
    if (tf > 0) {
      sel_f.ensure(tf - 1, lane, load_sel);
      mb = sel_f.at(tf - 1);
      if (mb < 0 || mb >= j) mb = 0;
    }
    const uint32_t so = (uint32_t)mb * (uint32_t)(kBlock * D * 2);
#pragma unroll
    for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Kh, kvbytes, kb + 512 * (wave + NW * i), voff[i], so);
#pragma unroll
    for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Vh, kvbytes, vb + 512 * (wave + NW * i), voff[i], so);
    if (tf < cnt_j) ++tf;
  };

  f32x16 oacc[D / 32][NTILE];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][nt][i] = 0.0f;
  float mref[NTILE], lrow[NTILE];
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) { mref[nt] = -INFINITY; lrow[nt] = 0.0f; }
  const float c2 = a.scale * kLog2e;

  // transposing-read addressing of V (see lds_tr16): lane (g, lp) supplies the address of
  // key 4*(g/2) + lp/4 (+ 8 for the second half) and d = 16*(g%2) + 4*(lp%4) of a 32 x 16 slab
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
    // Gate after the softmax: the logits and the normaliser are ungated (a block outside
    // S still drops out) and the probabilities are weighted by g before the PV product.
    const float gmul = OUT ? fast_exp2(lg2) : 1.0f;
    if (OUT) lg2 = ok ? 0.0f : -INFINITY;
    ++tc;
    fetch(kn, vn);
    if (!active) return;   // a missing head's waves only take part in the copies
    int rx = rx0, tx = tx0;
    asm volatile("" : "+v"(rx), "+v"(tx));   // keeps per-(buffer, read) addresses unhoisted
    f32x16 st[2][NTILE];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[mt][nt][i] = 0.0f;
    // S^T = K Q^T: the K operand reads go out in batches of 8 ahead of their products
#pragma unroll
    for (int k0 = 0; k0 < D / 16; k0 += 4) {
      bf16x8 kr[4][2];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) kr[u][mt] = as_bf16x8(ld16(&kc[32 * mt * D + (rx ^ ((k0 + u) << 4))]));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < NTILE; ++nt) st[mt][nt] = mfma32(kr[u][mt], qf[nt][k0 + u], st[mt][nt]);
    }
    // V^T operands of O^T += V^T P^T; with one row tile per wave they are read while the
    // softmax runs (two row tiles leave no registers for that)
    auto read_va = [&](int dt, int mt, int hh) {
      const int r0 = 32 * mt + 16 * hh;
      return join_tr16(lds_tr16(&vc[r0 * D + (tx ^ ((4 * dt) << 3))]),
                       lds_tr16(&vc[(r0 + 8) * D + (tx ^ ((4 * dt ^ 2) << 3))]));
    };
    bf16x8 va[D / 32][2][2];   // [dt][mt][hh]
    if constexpr (NTILE == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) va[dt][mt][hh] = read_va(dt, mt, hh);
    }
    if (DIAG) {  // causal mask on the current block (key > query)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTILE; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (key > wrow0 + 32 * nt + ql) st[mt][nt][i] = -INFINITY;
          }
    }
    // block maxima of the raw scores (scale > 0, so the max commutes with the affine map)
    float bmax[NTILE];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[mt][nt][i]);
      mx = half_max(mx);
      bmax[nt] = mx * c2 + lg2;
      grow |= bmax[nt] > mref[nt] + kRescaleThreshold;
    }
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt) {
        const float mnew = fmaxf(mref[nt], bmax[nt]);
        const float alpha = fast_exp2(mref[nt] - mnew);
        mref[nt] = mnew;
        lrow[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][nt][i] *= alpha;
      }
    }
    bf16x8 pf[2][NTILE][2];  // [mt][nt][half]
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) {
      const float off = lg2 - mref[nt];
      float ls = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(st[mt][nt][i] * c2 + off);
          st[mt][nt][i] = OUT ? p * gmul : p;
          ls += p;
        }
      lrow[nt] += ls;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int o = 8 * hh;
          pf[mt][nt][hh] = pack8(st[mt][nt][o], st[mt][nt][o + 1], st[mt][nt][o + 2], st[mt][nt][o + 3],
                                 st[mt][nt][o + 4], st[mt][nt][o + 5], st[mt][nt][o + 6], st[mt][nt][o + 7]);
        }
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 v = NTILE == 1 ? va[dt][mt][hh] : read_va(dt, mt, hh);
#pragma unroll
          for (int nt = 0; nt < NTILE; ++nt) oacc[dt][nt] = mfma32(v, pf[mt][nt][hh], oacc[dt][nt]);
        }
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
  wait_vm();   // the last (repeated) copy lands before the workgroup's LDS is released
  if (!active) return;

  const size_t lse_off = (size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock + wrow0;
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) {
    const float l = half_sum(lrow[nt]);
    const float inv = 1.0f / l;
    if (hl == 0) a.lse_rows[lse_off + 32 * nt + ql] = (mref[nt] + log2f(l)) * kLn2;
    const int qrow = 32 * nt + ql;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dt + 8 * g4 + 4 * hl;
        bf16x4 v;
        v[0] = (__bf16)(oacc[dt][nt][4 * g4 + 0] * inv);
        v[1] = (__bf16)(oacc[dt][nt][4 * g4 + 1] * inv);
        v[2] = (__bf16)(oacc[dt][nt][4 * g4 + 2] * inv);
        v[3] = (__bf16)(oacc[dt][nt][4 * g4 + 3] * inv);
        *reinterpret_cast<bf16x4*>(a.Oout + q_off + qrow * D + d0) = v;
      }
  }
}

template <int D, int NTILE, int NW, bool OUT>
static hipError_t launch_fwd_o(const AttnArgs& a, int nsplit, int hpw, hipStream_t st) {
  const int NB = a.n / kBlock;
  const unsigned grid = (unsigned)(NB * a.B * a.Hkv * nsplit);
  AttnArgs b = a;
  b.wg = wg_order(grid);
  ProfScope prof("fwd", st);
  hipLaunchKernelGGL((fwd_kernel<D, NTILE, NW, OUT>), dim3(grid), dim3(64 * NW), 0, st, b, nsplit, hpw);
  return hipGetLastError();
}

template <int D, int NTILE, int NW>
static hipError_t launch_fwd_t(const AttnArgs& a, int nsplit, int hpw, hipStream_t st) {
  if (a.gate_out) return launch_fwd_o<D, NTILE, NW, true>(a, nsplit, hpw, st);
  return launch_fwd_o<D, NTILE, NW, false>(a, nsplit, hpw, st);
}

// The same forward (32 rows per wave, two query heads per workgroup) at three waves per
// SIMD instead of two. Measured with rocprofv3's SQ counters, the two-wave kernel's waves
// spend ~43 % of their cycles waiting on instruction dependencies (LDS operands, matrix
// results) and the matrix cores overlap vector work in only ~39 % of their busy cycles; a
// third wave per SIMD covers more of those waits. That takes at most 168 registers per lane
// and 53 KB of LDS per workgroup: K stays double-buffered, V gets one buffer (48 KB in
// all), and the V^T operands are read just before their products (no register copy held
// across the softmax; 162 registers). Per step t:
//   copy V(t) into the V buffer and K(t+1) into the other K buffer;
//   S(t) from K(t); softmax(t);
//   wait for V(t) (K(t+1) may still be in flight), barrier; P V(t);
//   wait for K(t+1), barrier (every wave is done with V(t) and K(t) before they are refilled).
// The arithmetic and its order are those of fwd_kernel, so the outputs are identical.
template <int D, bool OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
void fwd3_kernel(const AttnArgs a, int nsplit, int hpw) {
  constexpr int NW = 4;
  constexpr int WPH = 2;
  __shared__ __attribute__((aligned(16))) uint16_t sk0[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sk1[Tile<D>::ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t sv[Tile<D>::ELEMS];
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
  const int head0 = split * hpw;
  const int nheads = min(hpw, G - head0);
  const int whead = wave / WPH;
  const int wrow0 = (wave % WPH) * 32;
  const bool active = whead < nheads;
  const int hq = h * G + head0 + (active ? whead : 0);
  const size_t kv_off = ((size_t)(b * a.Hkv + h) * a.n) * D;
  const uint16_t* Kh = a.K + kv_off;
  const uint16_t* Vh = a.V + kv_off;
  const size_t q_off = ((size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock + wrow0) * D;
  const size_t sel_row = (size_t)(b * a.Hkv + h) * NB + j;
  const int cnt_j = min(max(a.cnt[sel_row], 0), min(a.kcap, j));
  const int32_t* idx_row = a.idx + sel_row * a.kcap;
  const float* lg_row = a.logg != nullptr ? a.logg + sel_row * a.kcap : nullptr;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(ld16(a.Q + q_off + ql * D + 16 * ks + 8 * hl));
  auto load_sel = [&](int i, int& v, float& g) {
    v = i < cnt_j ? idx_row[i] : 0;
    g = (i < cnt_j && lg_row != nullptr) ? lg_row[i] * kLog2e : 0.0f;
  };
  LaneList sel_c, sel_k, sel_v;
  int tc = 0, tk = 0, tv = 0;
  constexpr int NWIN = Tile<D>::CPR / NW;
  uint32_t voff[NWIN];
#pragma unroll
  for (int i = 0; i < NWIN; ++i) {
    const int sidx = 64 * (wave + NW * i) + lane;
    const int rr = sidx / Tile<D>::CPR, c = sidx % Tile<D>::CPR;
    voff[i] = (uint32_t)(rr * D + ((c ^ Tile<D>::swz(rr)) << 3)) * 2u;
  }
  const int kvbytes = a.n * D * 2;
  auto block_of = [&](LaneList& L, int t) {
    int mb = j;
    if (t > 0) {
      L.ensure(t - 1, lane, load_sel);
      mb = L.at(t - 1);
      if (mb < 0 || mb >= j) mb = 0;
    }
    return (uint32_t)mb * (uint32_t)(kBlock * D * 2);
  };
  auto fetch_k = [&](uint16_t* kb) {
    const uint32_t so = block_of(sel_k, tk);
#pragma unroll
    for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Kh, kvbytes, kb + 512 * (wave + NW * i), voff[i], so);
    if (tk < cnt_j) ++tk;
  };
  auto fetch_v = [&]() {
    const uint32_t so = block_of(sel_v, tv);
#pragma unroll
    for (int i = 0; i < NWIN; ++i) buffer_load_lds16(Vh, kvbytes, sv + 512 * (wave + NW * i), voff[i], so);
    if (tv < cnt_j) ++tv;
  };
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

  auto step = [&](auto diag_c, const uint16_t* kc, uint16_t* kn) {
    constexpr bool DIAG = decltype(diag_c)::value;
    const int t = tc;
    float lg2 = 0.0f;
    bool ok = true;
    if (!DIAG) {
      sel_c.ensure(t - 1, lane, load_sel);
      const int mb = sel_c.at(t - 1);
      lg2 = sel_c.gat(t - 1);
      if (mb < 0 || mb >= j) { lg2 = -INFINITY; ok = false; }
    }
    const float gmul = OUT ? fast_exp2(lg2) : 1.0f;
    if (OUT) lg2 = ok ? 0.0f : -INFINITY;
    ++tc;
    fetch_v();        // V of this block (single buffer: every wave is done with the last one)
    fetch_k(kn);      // K of the next block (its buffer held block t - 1)
    int rx = rx0, tx = tx0;
    asm volatile("" : "+v"(rx), "+v"(tx));
    f32x16 st[2];
    if (active) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[mt][i] = 0.0f;
#pragma unroll
      for (int k0 = 0; k0 < D / 16; k0 += 4) {
        bf16x8 kr[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) kr[u][mt] = as_bf16x8(ld16(&kc[32 * mt * D + (rx ^ ((k0 + u) << 4))]));
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) st[mt] = mfma32(kr[u][mt], qf[k0 + u], st[mt]);
      }
      if (DIAG) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (key > wrow0 + ql) st[mt][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[mt][i]);
      mx = half_max(mx);
      const float bmax = mx * c2 + lg2;
      if (__any(bmax > mref + kRescaleThreshold)) {
        const float mnew = fmaxf(mref, bmax);
        const float alpha = fast_exp2(mref - mnew);
        mref = mnew;
        lrow *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
      }
    }
    bf16x8 pf[2][2];
    if (active) {
      const float off = lg2 - mref;
      float ls = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(st[mt][i] * c2 + off);
          st[mt][i] = OUT ? p * gmul : p;
          ls += p;
        }
      lrow += ls;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int o = 8 * hh;
          pf[mt][hh] = pack8(st[mt][o], st[mt][o + 1], st[mt][o + 2], st[mt][o + 3],
                             st[mt][o + 4], st[mt][o + 5], st[mt][o + 6], st[mt][o + 7]);
        }
    }
    wait_vm_n<NWIN>();   // V of this block has landed (the K copy behind it may not have)
    barrier_lds();
    if (active) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int r0 = 32 * mt + 16 * hh;
            const bf16x8 v = join_tr16(lds_tr16(&sv[r0 * D + (tx ^ ((4 * dt) << 3))]),
                                       lds_tr16(&sv[(r0 + 8) * D + (tx ^ ((4 * dt ^ 2) << 3))]));
            oacc[dt] = mfma32(v, pf[mt][hh], oacc[dt]);
          }
    }
    wait_vm();        // K of the next block has landed
    barrier_lds();    // ... for every wave, and every wave is done with sv and kc
  };
  const std::integral_constant<bool, true> diag_step;
  const std::integral_constant<bool, false> plain_step;
  fetch_k(sk0);
  wait_vm();
  barrier_lds();
  step(diag_step, sk0, sk1);
  const int nrest = cnt_j;
  const int nfull = nrest & ~1;
  for (int it = 0; it < nfull; it += 2) {
    step(plain_step, sk1, sk0);
    step(plain_step, sk0, sk1);
  }
  if (nfull < nrest) step(plain_step, sk1, sk0);
  wait_vm();
  if (!active) return;
  const size_t lse_off = (size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock + wrow0;
  const float l = half_sum(lrow);
  const float inv = 1.0f / l;
  if (hl == 0) a.lse_rows[lse_off + ql] = (mref + log2f(l)) * kLn2;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * dt + 8 * g4 + 4 * hl;
      bf16x4 v;
      v[0] = (__bf16)(oacc[dt][4 * g4 + 0] * inv);
      v[1] = (__bf16)(oacc[dt][4 * g4 + 1] * inv);
      v[2] = (__bf16)(oacc[dt][4 * g4 + 2] * inv);
      v[3] = (__bf16)(oacc[dt][4 * g4 + 3] * inv);
      *reinterpret_cast<bf16x4*>(a.Oout + q_off + ql * D + d0) = v;
    }
}

template <int D, bool OUT>
static hipError_t launch_fwd3_o(const AttnArgs& a, int nsplit, int hpw, hipStream_t st) {
  const int NB = a.n / kBlock;
  const unsigned grid = (unsigned)(NB * a.B * a.Hkv * nsplit);
  AttnArgs b = a;
  b.wg = wg_order(grid);
  ProfScope prof("fwd", st);
  hipLaunchKernelGGL((fwd3_kernel<D, OUT>), dim3(grid), dim3(256), 0, st, b, nsplit, hpw);
  return hipGetLastError();
}

// Heads of a KV group per workgroup: at most 4 waves of 64 rows; larger groups are split
// evenly across workgroups.
void head_split(int G, int* nsplit, int* hpw, int* nw) {
  *nsplit = (G + 3) / 4;
  *hpw = (G + *nsplit - 1) / *nsplit;
  *nw = *hpw <= 1 ? 1 : (*hpw <= 2 ? 2 : 4);
}

hipError_t launch_fwd(const AttnArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  int nsplit, hpw, nw;
  head_split(G, &nsplit, &hpw, &nw);
  if (G >= 2) {
    // 32 rows per wave (two waves per head), two heads per workgroup (split evenly)
    nsplit = (G + 1) / 2;
    hpw = (G + nsplit - 1) / nsplit;
    if (a.d == 128) return a.gate_out ? launch_fwd3_o<128, true>(a, nsplit, hpw, st)
                                      : launch_fwd3_o<128, false>(a, nsplit, hpw, st);
    return launch_fwd_t<64, 1, 4>(a, nsplit, hpw, st);
  }
  if (a.d == 128) {
    if (nw == 1) return launch_fwd_t<128, 2, 1>(a, nsplit, hpw, st);
    if (nw == 2) return launch_fwd_t<128, 2, 2>(a, nsplit, hpw, st);
    return launch_fwd_t<128, 2, 4>(a, nsplit, hpw, st);
  }
  if (nw == 1) return launch_fwd_t<64, 2, 1>(a, nsplit, hpw, st);
  if (nw == 2) return launch_fwd_t<64, 2, 2>(a, nsplit, hpw, st);
  return launch_fwd_t<64, 2, 4>(a, nsplit, hpw, st);
}

}  // namespace sas
