// Log-gated block-sparse attention forward on bf16 MFMA (gfx950).
//
// [SAS-ja] "仕組み", eq. (9) / [SAS-ko] "어떻게 동작하나": for query block j,
//   o = softmax(scale * q K_S^T + log g_S) V_S,  S = B_j (causal, gate 1) U the selected blocks,
// with log g of a selected block added to every logit of its 64 tokens. The gate add and
// the causal mask are fused into the logit tile; no attention matrix leaves registers.
//
// Work item: one workgroup per (batch, KV head, query block j[, head split]); each wave
// owns the 64 rows of one query head of the group, so one staged K/V block feeds
// G * 64 query rows (the GQA reuse that keeps the MFMA units fed).
//
// Orientation: each wave computes S^T = K Q^T (keys x queries) with 32x32x16 MFMAs. The
// accumulator then holds, per lane, one query column and 32 of its 64 keys, so the row
// softmax needs a single cross-lane exchange (lane ^ 32), and the probabilities are
// already laid out as the B operand of O^T += V^T P^T. V^T is staged in LDS with the key
// order permuted to match (perm32).
//
// Blocks are visited current block first, which makes every running row maximum finite
// from the start (each query sees at least itself), so -inf gates need no special case.
#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

template <int D>
struct FwdSmem {
  static constexpr int KP = D + 8;    // K row pitch (elements): conflict-free 16 B reads
  static constexpr int VP = 64 + 8;   // V^T row pitch (elements)
  uint16_t k[64 * KP];
  uint16_t vt[D * VP];
};

// Stage K (natural layout) and V^T (transposed, keys permuted) of one 64-token block.
template <int D, int NT>
__device__ __forceinline__ void stage_kv(FwdSmem<D>& sm, const uint16_t* Kb, const uint16_t* Vb,
                                         int tid) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int c = tid; c < 64 * CH; c += NT) {
    const int row = c / CH, col = c % CH;
    st16(&sm.k[row * FwdSmem<D>::KP + col * 8], ld16(Kb + row * D + col * 8));
  }
#pragma unroll
  for (int c = tid; c < 64 * CH; c += NT) {
    const int key = c & 63, col = c >> 6;
    const u16x8 v = ld16(Vb + key * D + col * 8);
    const int p = perm32(key);
#pragma unroll
    for (int e = 0; e < 8; ++e) sm.vt[(col * 8 + e) * FwdSmem<D>::VP + p] = v[e];
  }
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void fwd_kernel(const AttnArgs a, int nsplit, int hpw) {
  constexpr int NT = 64 * NW;
  __shared__ __attribute__((aligned(16))) FwdSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NB = a.n / kBlock, G = a.Hq / a.Hkv;

  // Heaviest query blocks first; consecutive workgroups differ in (split, head, batch) so
  // that a KV head stays on one XCD when B * Hkv * nsplit is a multiple of 8.
  const int per_j = a.B * a.Hkv * nsplit;
  const int j = NB - 1 - (int)(blockIdx.x / per_j);
  int r = blockIdx.x % per_j;
  const int split = r % nsplit;
  r /= nsplit;
  const int h = r % a.Hkv, b = r / a.Hkv;
  const int head0 = split * hpw;
  const int nheads = min(hpw, G - head0);
  const bool active = wave < nheads;
  const int hq = h * G + head0 + (active ? wave : 0);

  const size_t kv_off = ((size_t)(b * a.Hkv + h) * a.n) * D;
  const uint16_t* Kh = a.K + kv_off;
  const uint16_t* Vh = a.V + kv_off;
  const size_t q_off = ((size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock) * D;
  const size_t sel_row = (size_t)(b * a.Hkv + h) * NB + j;
  const int cnt_j = min(max(a.cnt[sel_row], 0), min(a.kcap, j));
  const int32_t* idx_row = a.idx + sel_row * a.kcap;
  const float* lg_row = a.logg != nullptr ? a.logg + sel_row * a.kcap : nullptr;

  // Q as the B operand of S^T = K Q^T: lane holds query 32*nt + l%32, d = 16*ks + 8*(l/32) + e.
  bf16x8 qf[2][D / 16];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qf[nt][ks] = active ? as_bf16x8(ld16(a.Q + q_off + (32 * nt + (lane & 31)) * D + 16 * ks + 8 * (lane >> 5)))
                          : bf16x8{};

  f32x16 oacc[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[dt][nt][i] = 0.0f;
  float mrow[2] = {-INFINITY, -INFINITY};
  float lrow[2] = {0.0f, 0.0f};
  const float c2 = a.scale * kLog2e;
  const int hl = lane >> 5, ql = lane & 31;

  for (int t = 0; t <= cnt_j; ++t) {
    int m = j;
    float lg2 = 0.0f;
    if (t > 0) {
      m = idx_row[t - 1];
      lg2 = lg_row != nullptr ? lg_row[t - 1] * kLog2e : 0.0f;
      if (m < 0 || m >= j) {  // ignored entry: stage block 0, weight 0
        m = 0;
        lg2 = -INFINITY;
      }
    }
    __syncthreads();
    stage_kv<D, NT>(sm, Kh + (size_t)m * kBlock * D, Vh + (size_t)m * kBlock * D, tid);
    __syncthreads();
    if (!active) continue;

    f32x16 st[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[mt][nt][i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 ka = as_bf16x8(ld16(&sm.k[(32 * mt + ql) * FwdSmem<D>::KP + 16 * ks + 8 * hl]));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) st[mt][nt] = mfma32(ka, qf[nt][ks], st[mt][nt]);
      }
    }
    // logits in base 2, gate, causal mask on the current block
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float z = st[mt][nt][i] * c2 + lg2;
          if (t == 0) {
            const int key = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (key > 32 * nt + ql) z = -INFINITY;
          }
          st[mt][nt][i] = z;
        }
    bf16x8 pf[2][2][2];  // [mt][nt][half]
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[mt][nt][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[nt], mx);
      const float alpha = exp2f(mrow[nt] - mnew);
      mrow[nt] = mnew;
      float ls = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = exp2f(st[mt][nt][i] - mnew);
          st[mt][nt][i] = p;
          ls += p;
        }
      lrow[nt] = lrow[nt] * alpha + ls;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][nt][i] *= alpha;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int o = 8 * hh;
          pf[mt][nt][hh] = pack8(st[mt][nt][o], st[mt][nt][o + 1], st[mt][nt][o + 2], st[mt][nt][o + 3],
                                 st[mt][nt][o + 4], st[mt][nt][o + 5], st[mt][nt][o + 6], st[mt][nt][o + 7]);
        }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 va = as_bf16x8(ld16(&sm.vt[(32 * dt + ql) * FwdSmem<D>::VP + 16 * (2 * mt + hh) + 8 * hl]));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) oacc[dt][nt] = mfma32(va, pf[mt][nt][hh], oacc[dt][nt]);
        }
  }
  if (!active) return;

  const size_t lse_off = (size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float l = lrow[nt] + __shfl_xor(lrow[nt], 32, 64);
    const float inv = 1.0f / l;
    if (hl == 0) a.lse_rows[lse_off + 32 * nt + ql] = (mrow[nt] + log2f(l)) * kLn2;
    const int qrow = 32 * nt + ql;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dt + 8 * g4 + 4 * hl;
        u16x4 v;
        v[0] = f2bf(oacc[dt][nt][4 * g4 + 0] * inv);
        v[1] = f2bf(oacc[dt][nt][4 * g4 + 1] * inv);
        v[2] = f2bf(oacc[dt][nt][4 * g4 + 2] * inv);
        v[3] = f2bf(oacc[dt][nt][4 * g4 + 3] * inv);
        *reinterpret_cast<u16x4*>(a.Oout + q_off + qrow * D + d0) = v;
      }
  }
}

template <int D, int NW>
static hipError_t launch_fwd_t(const AttnArgs& a, int nsplit, int hpw, hipStream_t st) {
  const int NB = a.n / kBlock;
  const unsigned grid = (unsigned)(NB * a.B * a.Hkv * nsplit);
  hipLaunchKernelGGL((fwd_kernel<D, NW>), dim3(grid), dim3(64 * NW), 0, st, a, nsplit, hpw);
  return hipGetLastError();
}

// Heads of a KV group per workgroup: at most 4 waves; larger groups are split evenly.
void head_split(int G, int* nsplit, int* hpw, int* nw) {
  *nsplit = (G + 3) / 4;
  *hpw = (G + *nsplit - 1) / *nsplit;
  *nw = *hpw <= 1 ? 1 : (*hpw <= 2 ? 2 : 4);
}

hipError_t launch_fwd(const AttnArgs& a, hipStream_t st) {
  int nsplit, hpw, nw;
  head_split(a.Hq / a.Hkv, &nsplit, &hpw, &nw);
  if (a.d == 128) {
    if (nw == 1) return launch_fwd_t<128, 1>(a, nsplit, hpw, st);
    if (nw == 2) return launch_fwd_t<128, 2>(a, nsplit, hpw, st);
    return launch_fwd_t<128, 4>(a, nsplit, hpw, st);
  }
  if (nw == 1) return launch_fwd_t<64, 1>(a, nsplit, hpw, st);
  if (nw == 2) return launch_fwd_t<64, 2>(a, nsplit, hpw, st);
  return launch_fwd_t<64, 4>(a, nsplit, hpw, st);
}

}  // namespace sas
