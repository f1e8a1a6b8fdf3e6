// Decode step in the inference form of SAS ([SAS-ja] "仕組み", Algorithm 2 / section 5.1):
// the new token of each sequence attends, without gates, to its current block plus the
// Top-K history blocks picked from s. Per (sequence, KV head) the G query heads share the
// selected K/V blocks, so each block is read from HBM once for all G heads.
//
// The work is HBM-bound. The block list of each (sequence, KV head) is split into chunks
// of `bpc` blocks so the launch has enough workgroups to fill 256 CUs; each workgroup
// writes a partial (running max, running sum, unnormalised output) per query head and a
// second kernel merges the partials with the usual log-sum-exp rescaling.
//
// Inside a workgroup (4 waves) wave w owns keys 16w..16w+15 of every block. A lane reads
// 16 contiguous bytes of one key row (coalesced rows), forms bf16 dot products with the G
// query heads held in registers, and reduces them across the lanes of its row.
#include "sas_common.h"
#include "sas_kernels.h"

namespace sas {

template <int D, int G>
__global__ __launch_bounds__(256) void decode_split_kernel(const DecodeArgs a) {
  constexpr int CPR = D / 8;      // lanes per key row (16 B each)
  constexpr int RPI = 64 / CPR;   // key rows per wave instruction
  constexpr int NI = 16 / RPI;    // instructions per wave per block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c8 = lane % CPR, rsub = lane / CPR;
  const int chunk = blockIdx.x % a.nchunk;
  const long long bh = blockIdx.x / a.nchunk;
  const int h = (int)(bh % a.Hkv), b = (int)(bh / a.Hkv);
  const int L = min(max(a.kv_len[b], 1), (int)a.Lmax);
  const int cur = (L - 1) / kBlock;
  const int cnt = min(max(a.cnt[bh], 0), min(a.kcap, cur));
  const int t0 = chunk * a.bpc, t1 = min(t0 + a.bpc, cnt + 1);
  const int32_t* idx_row = a.idx + bh * a.kcap;
  const float* lg_row = a.logg != nullptr ? a.logg + bh * a.kcap : nullptr;
  const size_t kv_base = (size_t)bh * a.Lmax * D;

  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const u16x8 v = ld16(a.q + ((size_t)b * a.Hq + h * G + g) * D + c8 * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[g][e] = bf2f(v[e]);
  }
  float mrun[G], lrun[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mrun[g] = -INFINITY;
    lrun[g] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
  }
  const float c2 = a.scale * kLog2e;

  for (int t = t0; t < t1; ++t) {
    int m = cur;
    float lg2 = 0.0f;
    if (t > 0) {
      m = idx_row[t - 1];
      lg2 = lg_row != nullptr ? lg_row[t - 1] * kLog2e : 0.0f;
      if (m < 0 || m >= cur) { m = 0; lg2 = -INFINITY; }
    }
    u16x8 kr[NI], vr[NI];
    int tok[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      tok[i] = m * kBlock + 16 * wave + RPI * i + rsub;
      const int tl = min(tok[i], (int)a.Lmax - 1);  // rows past the cache end are masked
      kr[i] = ld16(a.Kc + kv_base + (size_t)tl * D + c8 * 8);
      vr[i] = ld16(a.Vc + kv_base + (size_t)tl * D + c8 * 8);
    }
    float z[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = bf2f(kr[i][e]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s += qv[g][e] * kf[e];
#pragma unroll
        for (int off = CPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
        float zz = s * c2 + lg2;
        if (tok[i] >= L) zz = -INFINITY;
        z[i][g] = zz;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < NI; ++i) mx = fmaxf(mx, z[i][g]);
      mx = wave_max(mx);
      const float mnew = fmaxf(mrun[g], mx);
      if (mnew == -INFINITY) continue;  // nothing attendable yet
      const float alpha = exp2f(mrun[g] - mnew);
      mrun[g] = mnew;
      float ls = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float p = exp2f(z[i][g] - mnew);
        ls += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] += p * bf2f(vr[i][e]);
      }
      lrun[g] = lrun[g] * alpha + ls;
    }
  }

  // Sum over the key rows of the wave (lanes with the same c8), then merge the 4 waves.
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], off, 64);
      lrun[g] += __shfl_xor(lrun[g], off, 64);
    }
  }
  __shared__ float sm_m[4][G], sm_l[4][G];
  __shared__ float sm_acc[4][G][D];
  if (lane < CPR) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_acc[wave][g][c8 * 8 + e] = acc[g][e];
      if (lane == 0) { sm_m[wave][g] = mrun[g]; sm_l[wave][g] = lrun[g]; }
    }
  }
  __syncthreads();
  float* out = a.part + ((size_t)bh * a.nchunk + chunk) * G * (D + 2);
  for (int x = tid; x < G * D; x += 256) {
    const int g = x / D, dd = x % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][g]);
    float o = 0.0f, l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = exp2f(sm_m[w][g] - M);
        o += sc * sm_acc[w][g][dd];
        l += sc * sm_l[w][g];
      }
    }
    out[g * (D + 2) + 2 + dd] = o;
    if (dd == 0) { out[g * (D + 2)] = M; out[g * (D + 2) + 1] = l; }
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

template <int D, int G>
static void launch_split(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)((long long)a.B * a.Hkv * a.nchunk);
  hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(grid), dim3(256), 0, st, a);
}

template <int D>
static bool launch_split_g(const DecodeArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: launch_split<D, 1>(a, st); return true;
    case 2: launch_split<D, 2>(a, st); return true;
    case 4: launch_split<D, 4>(a, st); return true;
    case 5: launch_split<D, 5>(a, st); return true;
    case 8: launch_split<D, 8>(a, st); return true;
    default: return false;
  }
}

hipError_t launch_decode(DecodeArgs a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const long long pairs = (long long)a.B * a.Hkv;
  const int nblk = a.kcap + 1;
  // Aim for >= 2048 workgroups (8 per CU) without chunks of fewer than 2 blocks.
  int chunks = (int)((2048 + pairs - 1) / pairs);
  chunks = max(1, min(chunks, (nblk + 1) / 2));
  a.bpc = (nblk + chunks - 1) / chunks;
  a.nchunk = (nblk + a.bpc - 1) / a.bpc;
  const bool ok = a.d == 128 ? launch_split_g<128>(a, G, st) : launch_split_g<64>(a, G, st);
  if (!ok) return hipErrorInvalidValue;
  if (a.d == 128)
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((unsigned)(a.B * a.Hq)), dim3(128), 0, st, a);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace sas
