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
//   1. delta_t = dO_t . o_t                                  (HBM-bound row dots)
//   2. inverse index: for every key block m, the ascending list of (j, slot) with
//      idx[j][slot] = m, found by binary search in the ascending idx rows; the lists of
//      one (b, KV head) live in its own NB * kcap slice of the list buffer
//   3. query-major pass, one workgroup per (b, KV head, j): dQ and dg. dg_jm has exactly
//      one owner (the workgroup of j), reduced over its waves through LDS
//   4. key-major pass, one workgroup per (b, KV head, m): dK and dV over the current block
//      m itself plus every query block that selected m, all G heads
#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

void head_split(int G, int* nsplit, int* hpw, int* nw);

// ---------------------------------------------------------------- small kernels

__global__ void fill_f32_kernel(float* p, long long n, float v) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    p[i] = v;
}

template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const uint16_t* O, const uint16_t* dO,
                                                    float* delta, long long rows) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gid / LPR;
  const int c = (int)(gid % LPR);
  float acc = 0.0f;
  if (row < rows) {
    const u16x8 o = ld16(O + row * D + c * 8);
    const u16x8 g = ld16(dO + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += bf2f(o[e]) * bf2f(g[e]);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && c == 0) delta[row] = acc;
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

// Exclusive scan of the per-block counts of one (b, h): off[0..NB].
__global__ __launch_bounds__(256) void inv_scan_kernel(const int32_t* counts, int NB, int32_t* off) {
  __shared__ int32_t part[256];
  const long long bh = blockIdx.x;
  const int per = (NB + 255) / 256;
  const int t = threadIdx.x;
  int s = 0;
  for (int i = t * per; i < min(NB, (t + 1) * per); ++i) s += counts[bh * NB + i];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int run = part[t];
  for (int i = t * per; i < min(NB, (t + 1) * per); ++i) {
    off[bh * (NB + 1) + i] = run;
    run += counts[bh * NB + i];
  }
  if (t == 255) off[bh * (NB + 1) + NB] = run;
}

// ---------------------------------------------------------------- query-major: dQ, dg

template <int D>
struct DqSmem {
  static constexpr int KP = D + 8, TP = 64 + 8;
  uint16_t k[64 * KP];    // K natural (A operand of S^T = K Q^T)
  uint16_t kt[D * TP];    // K^T, keys permuted (A operand of dQ^T = K^T dS^T)
  uint16_t v[64 * KP];    // V natural (A operand of dP^T = V dO^T)
  float dgp[4];
};

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void dq_kernel(const AttnArgs a, int nsplit, int hpw) {
  constexpr int NT = 64 * NW, CH = D / 8;
  using SM = DqSmem<D>;
  __shared__ __attribute__((aligned(16))) SM sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, ql = lane & 31;
  const int NB = a.n / kBlock, G = a.Hq / a.Hkv;
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
  const size_t q_off = ((size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock) * D;
  const size_t row_off = (size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock;
  const size_t sel_row = (size_t)(b * a.Hkv + h) * NB + j;
  const int cnt_j = min(max(a.cnt[sel_row], 0), min(a.kcap, j));
  const int32_t* idx_row = a.idx + sel_row * a.kcap;
  const float* lg_row = a.logg != nullptr ? a.logg + sel_row * a.kcap : nullptr;
  float* dg_row = a.dg + sel_row * a.kcap;

  bf16x8 qf[2][D / 16], dof[2][D / 16];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const size_t o = q_off + (32 * nt + ql) * D + 16 * ks + 8 * hl;
      qf[nt][ks] = active ? as_bf16x8(ld16(a.Q + o)) : bf16x8{};
      dof[nt][ks] = active ? as_bf16x8(ld16(a.dO + o)) : bf16x8{};
    }
  float lse2[2], dl[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    lse2[nt] = active ? a.lse_rows[row_off + 32 * nt + ql] * kLog2e : 0.0f;
    dl[nt] = active ? a.delta[row_off + 32 * nt + ql] : 0.0f;
  }
  f32x16 dqacc[D / 32][2];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) dqacc[dt][nt][i] = 0.0f;
  const float c2 = a.scale * kLog2e;

  for (int t = 0; t <= cnt_j; ++t) {
    int m = j;
    float lg2 = 0.0f;
    bool ok = true;
    if (t > 0) {
      m = idx_row[t - 1];
      lg2 = lg_row != nullptr ? lg_row[t - 1] * kLog2e : 0.0f;
      if (m < 0 || m >= j) {
        m = 0;
        lg2 = -INFINITY;
        ok = false;
      }
    }
    __syncthreads();
    if (t >= 2 && tid == 0) {  // dg of the previous block, reduced over the waves
      float s = 0.0f;
      for (int w = 0; w < nheads; ++w) s += sm.dgp[w];
      if (nsplit == 1) dg_row[t - 2] = s; else atomicAdd(&dg_row[t - 2], s);
    }
    {
      const uint16_t* Kb = a.K + kv_off + (size_t)m * kBlock * D;
      const uint16_t* Vb = a.V + kv_off + (size_t)m * kBlock * D;
#pragma unroll
      for (int c = tid; c < 64 * CH; c += NT) {
        const int key = c & 63, col = c >> 6;
        const u16x8 kv = ld16(Kb + key * D + col * 8);
        st16(&sm.k[key * SM::KP + col * 8], kv);
        const int p = perm32(key);
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.kt[(col * 8 + e) * SM::TP + p] = kv[e];
        const int row = c / CH, cc = c % CH;
        st16(&sm.v[row * SM::KP + cc * 8], ld16(Vb + row * D + cc * 8));
      }
    }
    __syncthreads();
    if (!active) continue;

    f32x16 st[2][2], dpt[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) { st[mt][nt][i] = 0.0f; dpt[mt][nt][i] = 0.0f; }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 ka = as_bf16x8(ld16(&sm.k[(32 * mt + ql) * SM::KP + 16 * ks + 8 * hl]));
        const bf16x8 va = as_bf16x8(ld16(&sm.v[(32 * mt + ql) * SM::KP + 16 * ks + 8 * hl]));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          st[mt][nt] = mfma32(ka, qf[nt][ks], st[mt][nt]);
          dpt[mt][nt] = mfma32(va, dof[nt][ks], dpt[mt][nt]);
        }
      }
    const float gblk = exp2f(lg2);
    float dgacc = 0.0f;
    bf16x8 dsf[2][2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float zu = st[mt][nt][i] * c2;
          if (t == 0) {
            const int key = 32 * mt + 8 * (i >> 2) + 4 * hl + (i & 3);
            if (key > 32 * nt + ql) zu = -INFINITY;
          }
          const float u = exp2f(zu - lse2[nt]);
          const float dd = dpt[mt][nt][i] - dl[nt];
          dgacc += u * dd;
          ds[i] = u * gblk * dd;
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int o = 8 * hh;
          dsf[mt][nt][hh] = pack8(ds[o], ds[o + 1], ds[o + 2], ds[o + 3], ds[o + 4], ds[o + 5], ds[o + 6], ds[o + 7]);
        }
      }
    if (t > 0) {
      dgacc = ok ? wave_sum(dgacc) : 0.0f;
      if (lane == 0) sm.dgp[wave] = dgacc;
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const bf16x8 ka = as_bf16x8(ld16(&sm.kt[(32 * dt + ql) * SM::TP + 16 * (2 * mt + hh) + 8 * hl]));
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) dqacc[dt][nt] = mfma32(ka, dsf[mt][nt][hh], dqacc[dt][nt]);
        }
  }
  __syncthreads();
  if (tid == 0) {
    if (cnt_j >= 1) {
      float s = 0.0f;
      for (int w = 0; w < nheads; ++w) s += sm.dgp[w];
      if (nsplit == 1) dg_row[cnt_j - 1] = s; else atomicAdd(&dg_row[cnt_j - 1], s);
    }
  }
  if (split == 0)
    for (int p = cnt_j + tid; p < a.kcap; p += NT) dg_row[p] = 0.0f;
  if (!active) return;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * dt + 8 * g4 + 4 * hl;
        f32x4 v;
        v[0] = dqacc[dt][nt][4 * g4 + 0] * a.scale;
        v[1] = dqacc[dt][nt][4 * g4 + 1] * a.scale;
        v[2] = dqacc[dt][nt][4 * g4 + 2] * a.scale;
        v[3] = dqacc[dt][nt][4 * g4 + 3] * a.scale;
        *reinterpret_cast<f32x4*>(a.dQ + q_off + (32 * nt + ql) * D + d0) = v;
      }
}

// ---------------------------------------------------------------- key-major: dK, dV

template <int D>
struct DkvSmem {
  static constexpr int QP = D + 8, TP = 64 + 8;
  uint16_t q[64 * QP];    // Q_j natural   (A operand of S = Q K^T)
  uint16_t dob[64 * QP];  // dO_j natural  (A operand of dP = dO V^T)
  uint16_t qt[D * TP];    // Q_j^T, queries permuted (A operand of dK^T = Q^T dS)
  uint16_t dot[D * TP];   // dO_j^T        (A operand of dV^T = dO^T P)
  float lse2[64];
  float delta[64];
};

// Workgroup of 4 waves per (b, h, m); wave w owns keys 16w..16w+15 of block m with
// 16x16x32 MFMAs, so K and V of its keys stay in registers for the whole list.
template <int D>
__global__ __launch_bounds__(256) void dkv_kernel(const AttnArgs a) {
  using SM = DkvSmem<D>;
  constexpr int CH = D / 8;
  __shared__ __attribute__((aligned(16))) SM sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int NB = a.n / kBlock, G = a.Hq / a.Hkv;
  // Early key blocks are selected most often: launch them first.
  const int per_m = a.B * a.Hkv;
  const int m = (int)(blockIdx.x / per_m);
  const int r = blockIdx.x % per_m;
  const int h = r % a.Hkv, b = r / a.Hkv;
  const long long bh = (long long)b * a.Hkv + h;

  const size_t kv_off = ((size_t)bh * a.n + (size_t)m * kBlock) * D;
  const int key = 16 * wave + l16;  // this lane's key column within block m
  bf16x8 kf[D / 32], vf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    kf[ks] = as_bf16x8(ld16(a.K + kv_off + key * D + 32 * ks + 8 * g16));
    vf[ks] = as_bf16x8(ld16(a.V + kv_off + key * D + 32 * ks + 8 * g16));
  }
  f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) { dk[dt][i] = 0.0f; dv[dt][i] = 0.0f; }
  const float c2 = a.scale * kLog2e;
  const int off0 = a.inv_off[bh * (NB + 1) + m];
  const int nlist = a.inv_off[bh * (NB + 1) + m + 1] - off0;

  for (int e = 0; e <= nlist; ++e) {
    int j = m;
    float lg2 = 0.0f;
    if (e > 0) {
      const int p = a.inv_list[bh * NB * a.kcap + off0 + e - 1];
      j = p / a.kcap;
      const int slot = p - j * a.kcap;
      lg2 = a.logg != nullptr ? a.logg[((size_t)bh * NB + j) * a.kcap + slot] * kLog2e : 0.0f;
    }
    for (int g = 0; g < G; ++g) {
      const int hq = h * G + g;
      const size_t row0 = (size_t)(b * a.Hq + hq) * a.n + (size_t)j * kBlock;
      __syncthreads();
#pragma unroll
      for (int c = tid; c < 64 * CH; c += 256) {
        const int row = c & 63, col = c >> 6;
        const u16x8 qv = ld16(a.Q + (row0 + row) * D + col * 8);
        const u16x8 gv = ld16(a.dO + (row0 + row) * D + col * 8);
        st16(&sm.q[row * SM::QP + col * 8], qv);
        st16(&sm.dob[row * SM::QP + col * 8], gv);
        const int p = perm16(row);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          sm.qt[(col * 8 + x) * SM::TP + p] = qv[x];
          sm.dot[(col * 8 + x) * SM::TP + p] = gv[x];
        }
      }
      if (tid < 64) {
        sm.lse2[tid] = a.lse_rows[row0 + tid] * kLog2e;
        sm.delta[tid] = a.delta[row0 + tid];
      }
      __syncthreads();

      f32x4 s[4], dp[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) { s[qt][i] = 0.0f; dp[qt][i] = 0.0f; }
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const bf16x8 qa = as_bf16x8(ld16(&sm.q[(16 * qt + l16) * SM::QP + 32 * ks + 8 * g16]));
          const bf16x8 ga = as_bf16x8(ld16(&sm.dob[(16 * qt + l16) * SM::QP + 32 * ks + 8 * g16]));
          s[qt] = mfma16(qa, kf[ks], s[qt]);
          dp[qt] = mfma16(ga, vf[ks], dp[qt]);
        }
      float pv[4][4], dsv[4][4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = 16 * qt + 4 * g16 + i;
          float z = s[qt][i] * c2 + lg2;
          if (e == 0 && key > q) z = -INFINITY;
          const float p = exp2f(z - sm.lse2[q]);
          pv[qt][i] = p;
          dsv[qt][i] = p * (dp[qt][i] - sm.delta[q]);
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 pb = pack8(pv[2 * kk][0], pv[2 * kk][1], pv[2 * kk][2], pv[2 * kk][3],
                                pv[2 * kk + 1][0], pv[2 * kk + 1][1], pv[2 * kk + 1][2], pv[2 * kk + 1][3]);
        const bf16x8 sb = pack8(dsv[2 * kk][0], dsv[2 * kk][1], dsv[2 * kk][2], dsv[2 * kk][3],
                                dsv[2 * kk + 1][0], dsv[2 * kk + 1][1], dsv[2 * kk + 1][2], dsv[2 * kk + 1][3]);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const bf16x8 da = as_bf16x8(ld16(&sm.dot[(16 * dt + l16) * SM::TP + 32 * kk + 8 * g16]));
          const bf16x8 qa = as_bf16x8(ld16(&sm.qt[(16 * dt + l16) * SM::TP + 32 * kk + 8 * g16]));
          dv[dt] = mfma16(da, pb, dv[dt]);
          dk[dt] = mfma16(qa, sb, dk[dt]);
        }
      }
    }
  }
  float* dKp = a.dK + kv_off + key * D;
  float* dVp = a.dV + kv_off + key * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    const int d0 = 16 * dt + 4 * g16;
    f32x4 kv = dk[dt] * a.scale;
    *reinterpret_cast<f32x4*>(dKp + d0) = kv;
    *reinterpret_cast<f32x4*>(dVp + d0) = dv[dt];
  }
}

// ---------------------------------------------------------------- host side

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace_bytes(int B, int Hq, int Hkv, int n, int d, int kcap) {
  (void)d;
  const size_t NB = (size_t)n / kBlock;
  const size_t bh = (size_t)B * Hkv;
  return al256((size_t)B * Hq * n * sizeof(float))            // delta
         + al256(bh * NB * sizeof(int32_t))                    // counts
         + al256(bh * (NB + 1) * sizeof(int32_t))              // offsets
         + al256(bh * NB * (size_t)(kcap > 0 ? kcap : 1) * sizeof(int32_t));  // lists
}

template <int D>
static hipError_t launch_bwd_d(AttnArgs& a, hipStream_t st) {
  const int NB = a.n / kBlock;
  const long long nrows = (long long)a.B * a.Hkv * NB;
  const long long qrows = (long long)a.B * a.Hq * a.n;
  {
    const long long threads = qrows * (D / 8);
    hipLaunchKernelGGL(delta_kernel<D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                       a.Oout != nullptr ? a.Oout : a.O, a.dO, a.delta, qrows);
  }
  hipLaunchKernelGGL(inv_kernel, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, a.idx, a.cnt,
                     NB, a.kcap, nrows, a.inv_cnt, (const int32_t*)nullptr, (int32_t*)nullptr);
  hipLaunchKernelGGL(inv_scan_kernel, dim3((unsigned)(a.B * a.Hkv)), dim3(256), 0, st, a.inv_cnt, NB,
                     a.inv_off);
  hipLaunchKernelGGL(inv_kernel, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, a.idx, a.cnt,
                     NB, a.kcap, nrows, a.inv_cnt, (const int32_t*)a.inv_off, a.inv_list);
  int nsplit, hpw, nw;
  head_split(a.Hq / a.Hkv, &nsplit, &hpw, &nw);
  if (nsplit > 1) {
    const long long ndg = nrows * a.kcap;
    hipLaunchKernelGGL(fill_f32_kernel, dim3(1024), dim3(256), 0, st, a.dg, ndg, 0.0f);
  }
  const unsigned grid = (unsigned)nrows * nsplit;
  if (nw == 1) hipLaunchKernelGGL((dq_kernel<D, 1>), dim3(grid), dim3(64), 0, st, a, nsplit, hpw);
  else if (nw == 2) hipLaunchKernelGGL((dq_kernel<D, 2>), dim3(grid), dim3(128), 0, st, a, nsplit, hpw);
  else hipLaunchKernelGGL((dq_kernel<D, 4>), dim3(grid), dim3(256), 0, st, a, nsplit, hpw);
  hipLaunchKernelGGL(dkv_kernel<D>, dim3((unsigned)nrows), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd(AttnArgs a, void* ws, hipStream_t st) {
  const size_t NB = (size_t)a.n / kBlock;
  const size_t bh = (size_t)a.B * a.Hkv;
  char* p = (char*)ws;
  a.delta = (float*)p;
  p += al256((size_t)a.B * a.Hq * a.n * sizeof(float));
  a.inv_cnt = (int32_t*)p;
  p += al256(bh * NB * sizeof(int32_t));
  a.inv_off = (int32_t*)p;
  p += al256(bh * (NB + 1) * sizeof(int32_t));
  a.inv_list = (int32_t*)p;
  if (a.d == 128) return launch_bwd_d<128>(a, st);
  return launch_bwd_d<64>(a, st);
}

}  // namespace sas
