// Device helpers for the gfx950 kernels of libpagedattn.
//
// CDNA4 facts relied on: 64-lane wavefronts; DPP row operations act inside
// 16-lane rows; v_dot2_f32_bf16 multiplies two bf16 pairs and accumulates in
// fp32; v_exp_f32 computes 2^x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBlock = 16;          // tokens per cache block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f; // running-max start: finite, so 2^(m_old - m_new) never sees inf - inf
// Online softmax with a lazy reference: the running max only moves when a score
// exceeds it by more than this (base-2 units), so weights exp2(s - m) stay below
// 2^8 and accumulators are rarely rescaled.  l and acc always share one reference
// max, so the normalised result is the same softmax.
constexpr float kRescaleSlack = 8.0f;

// bf16 <-> fp32.  Stored bf16 is the upper half of the fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                          __builtin_bit_cast(bf16x2_t, b), c, false);
}

// DPP lane permutations inside 16-lane rows (all source lanes are in range).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xb1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4e;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over aligned groups of W consecutive lanes; every lane of a group gets the total.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(W == 8 || W == 16 || W == 32 || W == 64, "group width");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  if constexpr (W >= 16) x += dpp<kRowMirror>(x);
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Max / sum across lanes that differ only in bits >= log2(STRIDE) (i.e. across
// groups of STRIDE lanes); every lane gets the result.
template <int STRIDE>
__device__ __forceinline__ float cross_group_max(float x) {
#pragma unroll
  for (int off = STRIDE; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float cross_group_sum(float x) {
#pragma unroll
  for (int off = STRIDE; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float wave_max(float x) { return cross_group_max<1>(x); }
__device__ __forceinline__ float wave_sum(float x) { return cross_group_sum<1>(x); }

// 16-byte global load / store.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Element-type traits: bytes per element and elements per 16-byte chunk.
template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int bytes = 4; static constexpr int per16 = 4; };
template <> struct Elem<uint16_t> { static constexpr int bytes = 2; static constexpr int per16 = 8; };

__device__ __forceinline__ int clamp_block(int b, int num_blocks) {
  return (unsigned)b < (unsigned)num_blocks ? b : num_blocks - 1;
}

// Broadcast lane H of each 16-lane row to the whole row (DPP row_newbcast).
template <int H>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(H >= 0 && H < 16, "row lane");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + H, 0xf, 0xf, true));
}

// A buffer resource for `bytes` bytes at `base`, built in SGPRs; loads through
// it are bounds-checked against that range by the hardware.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, int voff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ---- Copies global -> LDS through the buffer unit ---------------------------

typedef __attribute__((address_space(3))) void lds_void_t;

// The copies into LDS below are waited for explicitly.  Vector memory
// operations complete in issue order, so "at most n outstanding" guarantees
// completion of every operation that has n or more younger ones.  The waits
// are assembly with a memory clobber so that no read of the copied data can
// be moved above them.
#define PA_VM_WAIT(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")

// Buffer resource words for `bytes` bytes at a wave-uniform `base`.
__device__ __forceinline__ u32x4_t rsrc_words(const uint8_t* base, int bytes) {
  const unsigned long long p = (unsigned long long)base;
  u32x4_t w;
  w.x = __builtin_amdgcn_readfirstlane((unsigned)p);
  w.y = __builtin_amdgcn_readfirstlane((unsigned)(p >> 32) & 0xffffu);
  w.z = __builtin_amdgcn_readfirstlane((unsigned)bytes);
  w.w = 0x00020000u;
  return w;
}

// Copy 16 bytes per lane from the buffer (lane offset `voff`, bounds-checked:
// out-of-range reads give zeros) to LDS at `lds` + 16 * lane.  Written as
// assembly so that the compiler does not track these copies: every read of
// the data they write is preceded by an explicit wait (PA_VM_WAIT), and extra
// operations it does not count only make its own waits stricter.  M0 holds
// the LDS address; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(u32x4_t rsrc, const void* lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void_t*)lds)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// As lds_copy16, with the non-temporal (nt) cache policy: the lines are
// fetched as a stream that the caches need not keep.  For data read once per
// launch (a decode's K/V tiles).  Measured on MI355X, batched decode (64
// sequences, 528 MB of K/V per launch): 99 -> 90.5 us; long context 0.74 ->
// 0.79 of HBM peak.  Where other sequences re-read the same blocks from the
// L2 (a shared prefix) it costs ~2%.
__device__ __forceinline__ void lds_copy16_nt(u32x4_t rsrc, const void* lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void_t*)lds)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// As lds_copy16, from a per-lane global address instead of a buffer
// resource (no bounds check: `src` must be valid for 16 bytes in every
// active lane).  For a few scattered rows, where building resources would
// cost scalar registers.
__device__ __forceinline__ void lds_copy16_global(const void* src, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void_t*)lds)), "v"(src)
               : "memory", "m0");
}
// As lds_copy16_global, 4 bytes per lane (to `lds` + 4 * lane).
__device__ __forceinline__ void lds_copy4_global(const void* src, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void_t*)lds)), "v"(src)
               : "memory", "m0");
}
// As lds_copy16, 4 bytes per lane (to `lds` + 4 * lane).
__device__ __forceinline__ void lds_copy4(u32x4_t rsrc, const void* lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void_t*)lds)), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most 8 * t vector memory operations (t tiles' copies) are outstanding, t = 1..3.
__device__ __forceinline__ void wait_tiles(int t) {
  if (t <= 1) PA_VM_WAIT(8);
  else if (t == 2) PA_VM_WAIT(16);
  else PA_VM_WAIT(24);
}
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;

// ds_read_b64_tr_b16: each lane reads 8 bytes (four bf16) at its own LDS
// address; within every group of 16 lanes the 4 x 16 block so read (lane l
// holding row l / 4, columns 4 (l % 4) .. +3) is handed back transposed, lane
// m of the group receiving column m's four values (rows 0..3).  With the four
// lanes of a row pointing at one key's 16 dims, lane m gets four keys of dim m:
// the A operand of a 16x16x16 MFMA whose k dimension is the keys.
__device__ __forceinline__ s16x4_t lds_read_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(lds_void_t*)p);
}

// Balanced split of a stream of `total` tiles over Wg ranks: rank r takes
// tiles [stream_start(r), stream_start(r + 1)).
__device__ __forceinline__ int64_t stream_start(int r, int64_t total, int Wg) { return (int64_t)r * total / Wg; }
// Rank whose range holds tile t: the largest r with stream_start(r) <= t.
__device__ __forceinline__ int stream_owner(int64_t t, int64_t total, int Wg) {
  return (int)(((t + 1) * Wg - 1) / total);
}

// Widen eight bf16 (one 16-byte chunk) to fp32.
__device__ __forceinline__ void widen_bf16x8(uint4 w, float* f) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x); f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z); f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

}  // namespace pa
