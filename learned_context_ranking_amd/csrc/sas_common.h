// Shared device helpers for the gfx950 kernels: vector types, MFMA wrappers, bf16
// conversion and wave-level reductions. Host code includes it only for the types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64;                 // tokens per block (the pages' b)
// word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle); out-of-range
// offsets read zero
constexpr int kBufferFlags = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-byte global / LDS accesses of raw bf16 bit patterns.
__device__ __forceinline__ u16x8 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u16x8*>(p);
}
__device__ __forceinline__ void st16(uint16_t* p, u16x8 v) {
  *reinterpret_cast<u16x8*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) { return __builtin_bit_cast(bf16x8, v); }

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l supplies A row l%32 and B column l%32 with the 8 k-values of half l/32; the
// accumulator element i of lane l is D[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(16x16) += A(16x32) * B(32x16); lane l supplies A row l%16 / B column l%16 with the
// 8 k-values of quarter l/16; accumulator element i of lane l is D[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 round-to-nearest-even (inputs here are finite).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Eight fp32 values to bf16 (round-to-nearest-even); pairs compile to v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4,
                                         float a5, float a6, float a7) {
  bf16x8 v;
  v[0] = (__bf16)a0; v[1] = (__bf16)a1; v[2] = (__bf16)a2; v[3] = (__bf16)a3;
  v[4] = (__bf16)a4; v[5] = (__bf16)a5; v[6] = (__bf16)a6; v[7] = (__bf16)a7;
  return v;
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes, lane l'
// receives element l'%4 of the 8-byte chunk addressed by lane 4e + l'/4, for e = 0..3.
// Used to read MFMA operands whose k-dimension is strided in LDS (V^T, K^T, Q^T, dO^T)
// from tiles stored in their natural row-major layout.
__device__ __forceinline__ i16x4 lds_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) uint16_t*)p));
}
__device__ __forceinline__ bf16x8 join_tr16(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// A 64-row tile of bf16 rows of D elements in LDS, unpadded (D*2 bytes per row) with the
// 16-byte chunks of row r stored at chunk position c ^ swz(r). The swizzle makes both
//  - row reads (16 lanes read the same chunk of 16 consecutive rows, ds_read_b128) and
//  - transposing reads (8 consecutive rows x 4 consecutive chunks, ds_read_b64_tr_b16)
// touch every LDS bank at most once / exactly twice, i.e. run without bank conflicts.
// Tiles are filled with global_load_lds (lane i of an instruction writes bytes
// [16 i, 16 i + 16) of a 1 KB window), so the swizzle is applied on the global side.
template <int D>
struct Tile {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int ELEMS = 64 * D;
  __device__ static __forceinline__ int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // element offset of (row r, element d)
  __device__ static __forceinline__ int off(int r, int d) {
    return r * D + ((((d >> 3) ^ swz(r))) << 3) + (d & 7);
  }
};

// Asynchronous global -> LDS copy of a 64-row tile whose rows are D elements apart in
// global memory. Wave w issues the 1 KB windows w, w + NW, ...; the per-lane source
// offsets depend only on (wave, lane), so they are computed once (TileLoader) and each
// copy adds a wave-uniform base. Completion is awaited with wait_vm() before the barrier
// that publishes the tile.
template <int D, int NW>
struct TileLoader {
  static constexpr int CPR = Tile<D>::CPR;
  static constexpr int N = CPR / NW;           // 1 KB windows per wave
  static_assert(CPR % NW == 0, "tile windows must split evenly over the waves");
  uint32_t off[N];                             // byte offset of this lane's 16 B in global memory
  int wave;
  __device__ __forceinline__ TileLoader(int wave_, int lane) : wave(wave_) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int s = 64 * (wave + NW * i) + lane;
      const int r = s / CPR, p = s % CPR;
      off[i] = (uint32_t)(r * D + ((p ^ Tile<D>::swz(r)) << 3)) * 2u;
    }
  }
  __device__ __forceinline__ void load(uint16_t* lds_tile, const uint16_t* g) const {
    const char* gb = (const char*)g;
#pragma unroll
    for (int i = 0; i < N; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(gb + off[i]),
                                       (__attribute__((address_space(3))) void*)(lds_tile + 512 * (wave + NW * i)),
                                       16, 0, 0);
  }
};
// Buffer loads straight into LDS: lane i of the wave copies 16 (or 4) bytes from
// base + voffset_i + soffset (soffset wave-uniform) to lds + 16 i (4 i). The buffer
// resource covers [base, base + bytes); reads beyond it return zero.
__device__ __forceinline__ void buffer_load_lds16(const void* base, int bytes, void* lds, uint32_t voffset,
                                                  uint32_t soffset) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, soffset, 0, 0);
}
__device__ __forceinline__ void buffer_load_lds4(const void* base, int bytes, void* lds, uint32_t voffset,
                                                 uint32_t soffset) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voffset, soffset, 0, 0);
}

// Wait until at most N vector-memory instructions of this wave are outstanding. Issued as
// the s_waitcnt intrinsic (not inline asm) so that the compiler's own wait insertion knows
// which copies have landed: otherwise it cannot tell that an LDS buffer filled by an
// earlier asynchronous copy is complete and waits for every copy in flight before reading it.
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vm() { wait_vm_n<0>(); }
// Workgroup barrier without the memory fence of __syncthreads(): that fence makes the
// compiler wait for every outstanding vector-memory instruction, including asynchronous
// tile copies meant to stay in flight across the barrier. Callers wait explicitly for the
// copies the next phase reads (wait_vm / wait_vm_n); LDS writes are drained here.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A wave-held window of a per-workgroup index list: lane i holds entry base + i, so entry
// t is read with a scalar readlane instead of a dependent memory load per step. Loaded 64
// entries at a time.
struct LaneList {
  int v = 0;
  float g = 0.0f;
  int base = -1;
  template <class F>
  __device__ __forceinline__ void ensure(int t, int lane, F&& load) {
    const int nb = t & ~63;
    if (nb != base) {
      base = nb;
      load(nb + lane, v, g);
      // vmcnt(0) as the intrinsic the compiler tracks: the refilled registers are ready on
      // this (rare) path, so no wait is needed where the paths merge (which would stall on
      // every tile copy in flight)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    }
  }
  __device__ __forceinline__ int at(int t) const { return __builtin_amdgcn_readlane(v, t & 63); }
  __device__ __forceinline__ float gat(int t) const {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), t & 63));
  }
};

// 2^x with the hardware v_exp_f32 (no denormal range reduction: results below 2^-126
// flush to zero, which is harmless for softmax weights relative to a maximum >= 1/256).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- Top-K of a wave's keys
// Selection compares fp32 scores through an order-preserving key (ties go to the lower
// block index, -0 equals +0 and NaN ranks as -inf before the key is formed). Lane l holds
// the keys of elements l + 64 i, i < nreg; padding keys are 0, below every valid key
// (order_key(-inf) = 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// inverse of order_key (exact for every key order_key produces)
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The cut of the k largest of `valid` keys (0 < k <= valid): keys above T are kept, and of
// the keys equal to T the need_eq lowest-index ones. T's 32 bits are fixed from the top: a
// candidate bit stays set when at least k keys are >= the candidate; the search stops once
// a candidate admits exactly k keys (then they are the kept set, whatever the lower bits).
// Whole wave. Two ways to count, same result:
//  * BALLOT = false: per-lane counts on the vector ALUs and one DPP wave reduction per bit,
//    for kernels that keep several waves on each SIMD (a ballot and a scalar popcount per
//    register would queue them all on the CU's single scalar unit);
// Either way the registers past the row's keys (i >= nreg) must hold 0: the counts run
// over a compile-time number of registers, the smallest listed step >= nreg.
//  * BALLOT = true: one compare mask per register, summed by scalar popcounts, for a wave
//    that has its SIMD to itself (no reduction chain: the latency of each bit is a few
//    issue slots).
template <int PL, bool BALLOT = false>
__device__ __forceinline__ void topk_cut(const uint32_t (&key)[PL], int nreg, int valid, int k, uint32_t& T,
                                         int& need_eq);
// Calls f(i, pos) for every kept register i of this lane, pos its slot in index order
// (ascending element index: a ballot prefix count, no sort). Fully unrolled whatever its
// size: a rolled loop would index the key registers and put them in scratch memory.
template <int PL, class F>
__device__ __forceinline__ void topk_walk(const uint32_t (&key)[PL], int nreg, uint32_t T, int need_eq, F&& f) {
  const int lane = threadIdx.x & 63;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int base = 0, eq_before = 0;
  if (need_eq == 0) {   // no key equal to T is kept (the usual case): one ballot per register
#pragma clang loop unroll(full)
    for (int i = 0; i < PL; ++i) {
      if (i < nreg) {
        const bool sel = key[i] > T;
        const unsigned long long bsel = __ballot(sel);
        if (sel) f(i, base + __popcll(bsel & lt));
        base += __popcll(bsel);
      }
    }
    return;
  }
#pragma clang loop unroll(full)
  for (int i = 0; i < PL; ++i) {
    if (i < nreg) {   // (a guard, not a break: a constant trip count unrolls in full)
      const bool eq = key[i] == T;
      const unsigned long long beq = __ballot(eq);
      const int eq_rank = eq_before + __popcll(beq & lt);
      const bool sel = key[i] > T || (eq && eq_rank < need_eq);
      const unsigned long long bsel = __ballot(sel);
      if (sel) f(i, base + __popcll(bsel & lt));
      base += __popcll(bsel);
      eq_before += __popcll(beq);
    }
  }
}

// The walk for a cut that keeps no key equal to T (need_eq == 0), without branches: calls
// f(i, pos, kept) for every register i < NR of this lane, pos the key's slot in index order
// when kept (the compare's lane mask, counted below the lane and carried across registers
// by scalar popcounts). The registers past nreg must hold 0.
template <int NR, int PL, class F>
__device__ __forceinline__ void topk_walk_gt(const uint32_t (&key)[PL], uint32_t T, F&& f) {
  constexpr int kUGT = 34;   // integer compare predicate: unsigned >
  int base = 0;
#pragma clang loop unroll(full)
  for (int i = 0; i < NR; ++i) {
    const unsigned long long m = __builtin_amdgcn_uicmp(key[i], T, kUGT);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    f(i, base + below, key[i] > T);
    base += __builtin_popcountll(m);
  }
}

// Max / sum of a lane's value and that of lane l ^ 32, in every lane. v_permlane32_swap
// exchanges the two 32-lane halves between two copies of the value (a vector-ALU
// instruction; __shfl_xor(v, 32) is an LDS permute), so each lane then holds the pair
// {v_l, v_(l^32)}, and both halves get the same result.
__device__ __forceinline__ float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide reductions through DPP lane moves, register to register (a butterfly of
// __shfl_xor compiles to LDS permutes, one round trip each). An inclusive scan within each
// row of 16 lanes by row shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row
// contribute the identity), then the row totals carried forward by the broadcasts of lane
// 15 (into rows 1 and 3) and lane 31 (into rows 2 and 3): lane 63 ends with the total,
// which is returned as a wave-uniform value. All 64 lanes must be active.
template <class Op>
__device__ __forceinline__ int dpp_reduce(int v, int identity, Op op) {
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x111, 0xf, 0xf, false));   // row_shr:1
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x112, 0xf, 0xf, false));   // row_shr:2
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x114, 0xf, 0xf, false));   // row_shr:4
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x118, 0xf, 0xf, false));   // row_shr:8
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x142, 0xa, 0xf, false));   // row_bcast:15
  v = op(v, __builtin_amdgcn_update_dpp(identity, v, 0x143, 0xc, 0xf, false));   // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int dpp_sum_i(int v) {
  return dpp_reduce(v, 0, [](int x, int y) { return x + y; });
}
__device__ __forceinline__ float dpp_sum(float v) {
  return __int_as_float(dpp_reduce(__float_as_int(v), 0,
                                   [](int x, int y) { return __float_as_int(__int_as_float(x) + __int_as_float(y)); }));
}
__device__ __forceinline__ float dpp_max(float v) {
  return __int_as_float(dpp_reduce(__float_as_int(v), __float_as_int(-INFINITY),
                                   [](int x, int y) { return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y))); }));
}

// Number of keys >= c (GE) or > c over the wave's first NR registers: per-lane counts on
// the vector ALUs (a compare and an add each; no guard per register, whose lane-mask
// combination would cost two more instructions) and one DPP wave reduction. Registers
// past the row's keys must hold 0.
template <int NR, int PL, bool GE>
__device__ __forceinline__ int topk_count_dpp(const uint32_t (&key)[PL], uint32_t c) {
  int cl = 0;
#pragma clang loop unroll(full)
  for (int i = 0; i < NR; ++i) cl += (GE ? key[i] >= c : key[i] > c) ? 1 : 0;
  return dpp_sum_i(cl);
}
// The same over the first NR registers, each compare's lane mask (v_cmp into a scalar
// register pair) summed by scalar popcounts. No guard per register (it would be a branch
// each): registers i >= nreg must hold 0, which is never > c and never >= a candidate
// (candidates have a bit set).
template <int NR, int PL, bool GE>
__device__ __forceinline__ int topk_count_mask(const uint32_t (&key)[PL], uint32_t c) {
  constexpr int kUGE = 35, kUGT = 34;   // integer compare predicates (unsigned >=, >)
  int n = 0;
#pragma clang loop unroll(full)
  for (int i = 0; i < NR; ++i) n += __builtin_popcountll(__builtin_amdgcn_uicmp(key[i], c, GE ? kUGE : kUGT));
  return n;
}

template <int PL, int NR, bool BALLOT>
__device__ __forceinline__ void topk_cut_n(const uint32_t (&key)[PL], int nreg, int valid, int k, uint32_t& T,
                                           int& need_eq) {
  auto count = [&](uint32_t c, auto ge) {
    if constexpr (BALLOT) return topk_count_mask<NR, PL, decltype(ge)::value>(key, c);
    else return topk_count_dpp<NR, PL, decltype(ge)::value>(key, c);
  };
  T = 0;
  if (k < valid) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      const int c = count(cand, std::true_type{});
      if (c >= k) {
        T = cand;
        if (c == k) { T = cand - 1u; break; }   // the kept set: the keys > cand - 1, no ties
      }
    }
  }
  // (k == valid keeps every valid key: T = 0 is below all of them)
  need_eq = k - count(T, std::false_type{});
}

template <int PL, bool BALLOT>
__device__ __forceinline__ void topk_cut(const uint32_t (&key)[PL], int nreg, int valid, int k, uint32_t& T,
                                         int& need_eq) {
  // count over the smallest compile-time number of registers that holds the row's keys
  // (a half or all of them with mask counts, a quarter steps with per-lane counts)
  if constexpr (BALLOT && PL >= 2) {
    if (nreg <= PL / 2) topk_cut_n<PL, PL / 2, true>(key, nreg, valid, k, T, need_eq);
    else topk_cut_n<PL, PL, true>(key, nreg, valid, k, T, need_eq);
  } else if constexpr (!BALLOT && PL >= 8) {
    if (nreg <= PL / 4) topk_cut_n<PL, PL / 4, false>(key, nreg, valid, k, T, need_eq);
    else if (nreg <= PL / 2) topk_cut_n<PL, PL / 2, false>(key, nreg, valid, k, T, need_eq);
    else if (nreg <= 3 * PL / 4) topk_cut_n<PL, 3 * PL / 4, false>(key, nreg, valid, k, T, need_eq);
    else topk_cut_n<PL, PL, false>(key, nreg, valid, k, T, need_eq);
  } else {
    topk_cut_n<PL, PL, BALLOT>(key, nreg, valid, k, T, need_eq);
  }
}

// Position of key k within its 16-key group when a transposed operand is staged in LDS
// so that each lane's 8 MFMA k-values are contiguous: a 32x32x16 accumulator gives lane
// half h the keys {4h..4h+3, 8+4h..8+4h+3}; swapping bits 2 and 3 of the key makes them
// positions 8h..8h+7.
__device__ __forceinline__ int perm32(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}
// The same for the 16x16x32 accumulator pairs used by the key-major backward: within a
// 32-query group, query q' = 16a + 4g + r (a<2, g<4, r<4) is stored at 8g + 4a + r.
__device__ __forceinline__ int perm16(int q) {
  return (q & ~31) | (((q >> 2) & 3) << 3) | (((q >> 4) & 1) << 2) | (q & 3);
}

}  // namespace sas
