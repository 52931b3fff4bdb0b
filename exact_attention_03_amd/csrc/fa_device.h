// fa_device.h - gfx950 device primitives shared by the attention kernels.
//
// MFMA tiles, bounds-checked buffer loads/stores, swizzled LDS tile layout,
// transposed LDS reads and the cross-half lane exchange.  The lane layouts
// below are those of the CDNA4 matrix instructions:
//
//   v_mfma_f32_32x32x16_{f16,bf16}:  A is 32(m) x 16(k), B is 16(k) x 32(n).
//   Lane l (h = l/32) supplies A[m = l%32][k in K_h] and B[k in K_h][n = l%32],
//   eight k values per lane, the same set K_h for A and B.  Because the k index
//   is summed, which eight k's a half supplies is a free choice as long as A and
//   B agree; this library always feeds k = 8h + i (i = 0..7) of each 16-wide k
//   step.  The 32x32 fp32 result lands in 16 registers per lane:
//   register j of lane l holds C[m = 8(j/4) + 4h + j%4][n = l%32].
//
// Row permutation sigma.  When the A rows of a 32-row block are loaded in the
// order sigma(m) (bits 2 and 3 of m swapped), register j of the result holds
// row 16(j/8) + 8h + (j%8): the first eight registers are eight consecutive
// rows and so are the last eight.  That makes a score tile directly usable as
// the k-operand of the next MFMA (eight consecutive keys per lane half) and
// lets results be stored as 16-byte vectors.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

#define FA_DEV __device__ __forceinline__
#define FA_HD __host__ __device__ __forceinline__

// An empty statement the compiler must not execute speculatively: placed in a
// rarely taken uniform branch it keeps the branch from being flattened into
// per-element selects that every iteration would pay for.
FA_DEV void keep_branch() { asm volatile("" ::: "memory"); }

// Index of the calling wave in its workgroup, as a scalar: the compiler then
// treats everything derived from it (per-wave key or query ranges, mask
// decisions) as wave-uniform, keeping it in SGPRs and branching on it.
FA_DEV int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Element-type tags.
struct F16 {
  static constexpr int code = 0;
};
struct BF16 {
  static constexpr int code = 1;
};
struct F32 {
  static constexpr int code = 2;
};

template <typename T>
inline constexpr bool kIsBF16 = false;
template <>
inline constexpr bool kIsBF16<BF16> = true;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ----------------------------------------------------------------- MFMA
template <typename T>
FA_DEV f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
FA_DEV f32x16 mfma32<F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
FA_DEV f32x16 mfma32<BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 values to one dword of two 16-bit values, round to nearest even.
// v_mfma_f32_16x16x32_{f16,bf16} (A 16(m) x 32(k), B 32(k) x 16(n)) and
// v_mfma_f32_16x16x16_{f16,bf16} (k = 16).  Lane l (g = l/16) supplies
// A[m = l%16][k in K_g] and B[k in K_g][n = l%16], the same set K_g for A and
// B (this library feeds k = 8g + i, i = 0..7, and k = 4g + i, i = 0..3); the
// 16x16 fp32 result lands in 4 registers per lane: register i of lane l holds
// C[m = 4g + i][n = l%16].  That is the B-operand layout of a k = 16 product,
// so a result can feed the next product as its B operand directly.
template <typename T>
FA_DEV f32x4 mfma16k32(u32x4 a, u32x4 b, f32x4 c);
template <>
FA_DEV f32x4 mfma16k32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
template <>
FA_DEV f32x4 mfma16k32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <typename T>
FA_DEV f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c);
template <>
FA_DEV f32x4 mfma16k16<F16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                               0);
}
template <>
FA_DEV f32x4 mfma16k16<BF16>(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                   0, 0, 0);
}

template <typename T>
FA_DEV uint32_t pack2(float a, float b);
template <>
FA_DEV uint32_t pack2<F16>(float a, float b) {
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
template <>
FA_DEV uint32_t pack2<BF16>(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Registers [j0, j0+8) of an accumulator tile packed into an MFMA operand.
template <typename T>
FA_DEV u32x4 pack8(const f32x16& s, int j0) {
  u32x4 r;
  r.x = pack2<T>(s[j0 + 0], s[j0 + 1]);
  r.y = pack2<T>(s[j0 + 2], s[j0 + 3]);
  r.z = pack2<T>(s[j0 + 4], s[j0 + 5]);
  r.w = pack2<T>(s[j0 + 6], s[j0 + 7]);
  return r;
}

// 16-bit storage value back to fp32 (for the preprocess pass).
template <typename T>
FA_DEV float lo16_to_f32(uint32_t w);
template <typename T>
FA_DEV float hi16_to_f32(uint32_t w);
template <>
FA_DEV float lo16_to_f32<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <>
FA_DEV float hi16_to_f32<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <>
FA_DEV float lo16_to_f32<BF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <>
FA_DEV float hi16_to_f32<BF16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// ----------------------------------------------------------------- lanes
FA_HD int sigma32(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }
// Swap bits 0 and 1: sigma restricted to the 4-element chunk index of a 16-lane group.
FA_HD int swap01(int c) { return (c & ~3) | ((c & 1) << 1) | ((c & 2) >> 1); }

// {x of this lane, x of lane l^32}: max / sum across the two lane halves.
FA_DEV float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
FA_DEV float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

FA_DEV bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

FA_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ----------------------------------------------------------------- global memory
// Buffer resources give hardware bounds checks: loads past num_records return
// zero and stores past it are dropped.  Every kernel builds its resources over
// one head (N*D elements), so a ragged last tile needs no extra guards.
constexpr int kBufferFlags = 0x00020000;  // gfx9 raw-buffer data format word

FA_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferFlags);
}
FA_DEV u32x4 gload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
FA_DEV void gstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
FA_DEV float gload_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
FA_DEV void gstore_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
FA_DEV u32x2 gload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

// Global -> LDS copy without a register round trip (gfx950 16-byte buffer
// load into LDS): lane l's 16 bytes at byte offset voff of the resource land
// at lds_base + 16 l.  lds_base must be the same for the whole wave.  Bytes
// past the resource's end arrive as zeros.  Completion is tracked by vmcnt.
typedef __attribute__((address_space(3))) void lds_void_t;
FA_DEV void dma16(__amdgpu_buffer_rsrc_t r, char* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 16, voff, 0, 0, 0);
}
// The same with 4 bytes per lane: lane l's dword lands at lds_base + 4 l.
FA_DEV void dma4(__amdgpu_buffer_rsrc_t r, char* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_base, 4, voff, 0, 0, 0);
}
// Wait until every global load of this wave (including LDS copies) is done.
// Emitted through the builtin (s_waitcnt with vmcnt 0 and the other counters
// at their maximum), not inline assembly, so that the compiler's own wait
// insertion knows every earlier load has completed and adds no further waits
// for registers loaded before this point.  The builtin does not order memory
// accesses for the compiler: every use is followed by __syncthreads(), which
// does, before any LDS read of the copied data.
FA_DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ----------------------------------------------------------------- LDS tiles
// A tile of R rows x D 16-bit elements (D a multiple of 32) is stored in LDS
// as D/32 column groups; group G holds chunks 4G .. 4G+3 (16 bytes = 8
// elements each) of every row, 64 bytes per row, rows in order, and inside a
// row chunk 4G + j sits at position j ^ ((row / 4) % 4).
//  * 16-byte reads of one chunk by 16 lanes whose rows are a permutation of an
//    aligned block of 16 rows: row % 4 picks the 64-byte quarter of the
//    256-byte bank window and (row / 4) % 4 the 16-byte position in it, so the
//    16 reads hit each bank once.
//  * transposing 8-byte reads, where 32 lanes read 4 consecutive rows x the 4
//    chunks of one group: 4 rows x 64 bytes, each bank once.
//  * the swizzle only depends on bits 2-3 of the row, which the loops never
//    vary, so every address the matrix loops need is one of two per-lane bases
//    plus a compile-time offset: the loops do no address arithmetic.
//  * global -> LDS copies fill the slots in order: a 1 KiB copy covers 16 rows
//    x 64 contiguous bytes of the source.
template <int R>
struct CmTile {
  static_assert(R % 16 == 0, "tiles are whole 16-row blocks");
  static constexpr int GB = R * 64;  // bytes per group of 4 chunks
  FA_HD static int swz(int row) { return (row >> 2) & 3; }
  FA_HD static int off(int row, int chunk) {
    return (chunk >> 2) * GB + row * 64 + (((chunk & 3) ^ swz(row)) << 4);
  }
  // Slot s (the 16 bytes at 16 s) holds (slot_row(s), slot_chunk(s)).
  FA_HD static int slot_row(int s) { return (s >> 2) % R; }
  FA_HD static int slot_chunk(int s) { return 4 * (s / (4 * R)) + ((s & 3) ^ swz(slot_row(s))); }
};

FA_DEV u32x4 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// 16-byte operand reads of row `row` at k step t (chunk 2t + h):
// at(t) = base[t % 2] + (t / 2) GB.  Rows 32 b + row of other 32-row blocks
// are 2048 b bytes further on.
template <int R>
struct RowRead {
  int b0, b1;
  FA_HD RowRead(int row, int h) : b0(CmTile<R>::off(row, h)), b1(CmTile<R>::off(row, 2 + h)) {}
  FA_HD int at(int t) const { return ((t & 1) ? b1 : b0) + (t >> 1) * CmTile<R>::GB; }
};
constexpr int kRowBlockBytes = 32 * 64;  // one 32-row block of a tile

// Transposed 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i%4) of the 8-byte chunks fetched by lanes
// 4r + i/4 of its group, r = 0..3, as its elements r = 0..3.
FA_DEV u32x2 lds_read_tr(const char* base, int off) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
  return __builtin_bit_cast(u32x2, v);
}

// Per-lane bases of the transposing operand reads below.  Lane (g = group of
// 16, r = (lane % 16) / 4, c = lane % 4) fetches 4 elements of row
// 8h + r (and 8h + 4 + r) at column 16 (g % 2) + 4 swap01(c) of a 32-column
// block.
template <int R>
struct TrRead {
  int lo, hi;
  FA_HD explicit TrRead(int lane) {
    const int g = lane >> 4, h = lane >> 5, r = (lane & 15) >> 2, c = swap01(lane & 3);
    const int x = 2 * (g & 1) + (c >> 1);  // chunk within the 32-column block
    const int e = 4 * (c & 1);              // first element within the chunk
    lo = CmTile<R>::off(8 * h + r, x) + 2 * e;
    hi = CmTile<R>::off(8 * h + 4 + r, x) + 2 * e;
  }
};

// MFMA operand of 8 consecutive k (tile rows k0 + 8h .. k0 + 8h + 7 for lane
// half h; k0 a multiple of 16) for the 32-column block db, where the 32 operand
// lanes take the columns in sigma order: lane l receives
// T[k0 + 8h + i][32 db + sigma(l % 32)] for i = 0..7.
template <int R>
FA_DEV u32x4 lds_read_tr_operand(const char* tile, const TrRead<R>& b, int k0, int db) {
  const int o = k0 * 64 + db * CmTile<R>::GB;
  const u32x2 lo = lds_read_tr(tile, b.lo + o);
  const u32x2 hi = lds_read_tr(tile, b.hi + o);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Transposed operand of a 16x16x32 product with the contraction index along
// tile rows: lane l (g = l / 16) receives T[k0 + 8g + i][c0 + l % 16] for
// i = 0..7 (k0, c0 multiples of 16), the A layout A[m = l % 16][k = 8g + i]
// (or the B layout B[k = 8g + i][n = l % 16]) with m (n) = column
// c0 + l % 16.  Two transposing reads: fetching lane 16g + 4r + c takes the 8
// bytes at row k0 + 8g + r (then 8g + 4 + r), columns c0 + 4c .. c0 + 4c + 3;
// lanes 0-31 (and 32-63) then cover rows of two swizzle classes, each bank
// once.  The lane-dependent part of an address only depends on the parity of
// c0 / 16 and on which of the two reads it is, so a lane keeps four bases (in
// named registers: an indexed array would be placed in LDS) and every read is
// a base plus a compile-time offset.
template <int R>
struct TrRead16 {
  int b00, b01, b10, b11;  // b<parity of c0 / 16><first / second read>
  FA_HD static int base(int lane, int e, int x) {
    const int g = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
    // column 16 e + 4 c of a 32-column group lies in chunk 2 e + c / 2
    return CmTile<R>::off(8 * g + 4 * x + r, 2 * e + (c >> 1)) + 8 * (c & 1);
  }
  FA_HD explicit TrRead16(int lane)
      : b00(base(lane, 0, 0)), b01(base(lane, 0, 1)), b10(base(lane, 1, 0)), b11(base(lane, 1, 1)) {}
};
template <int R>
FA_DEV u32x4 lds_read_tr16(const char* tile, const TrRead16<R>& t, int k0, int c0) {
  const bool odd = (c0 >> 4) & 1;
  const int o = k0 * 64 + (c0 >> 5) * CmTile<R>::GB;
  const u32x2 lo = lds_read_tr(tile, (odd ? t.b10 : t.b00) + o);
  const u32x2 hi = lds_read_tr(tile, (odd ? t.b11 : t.b01) + o);
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

FA_DEV void gstore8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

}  // namespace fa
