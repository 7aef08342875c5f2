// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vl {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Lane l holds A[row l%32][k 8*(l/32) .. +8], B[k 8*(l/32) .. +8][col l%32];
// C value v of lane l is C[row 8*(v/4) + 4*(l/32) + v%4][col l%32].
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) {
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ u32x4 as_u32x4(const bf16x8& b) {
  return __builtin_bit_cast(u32x4, b);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Row index permutation of the 32-row A operand that makes the C rows held by
// lane half h for k-step s (C values 8s .. 8s+7) the consecutive keys
// 16s + 8h + 0..7: swap bits 2 and 3.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Row-major bf16 tile of D columns in LDS.  The 16-byte chunks of a row are
// XOR-swizzled with the row index (its two 2-bit fields swapped) so that
//  * 16 lanes reading one chunk of 16 consecutive rows (ds_read_b128),
//  * 16 lanes writing the 16 chunks of one row, and
//  * a transpose read (ds_read_b64_tr_b16) of 4 rows x 32 columns by 32 lanes
// all touch distinct banks.
template <int D>
struct SwzTile {
  static constexpr int NCH = D / 8;  // chunks per row
  __device__ __forceinline__ static int swz(int row) {
    return (((row & 3) << 2) | ((row >> 2) & 3)) & (NCH - 1);
  }
  // element offset of 16-byte chunk `ch` of `row`
  __device__ __forceinline__ static int chunk(int row, int ch) {
    return row * D + ((ch ^ swz(row)) << 3);
  }
  // element offset of column `col` (col % 4 == 0 for 8-byte accesses)
  __device__ __forceinline__ static int elem(int row, int col) {
    return row * D + (((col >> 3) ^ swz(row)) << 3) + (col & 7);
  }
};

typedef __attribute__((ext_vector_type(4))) short s16x4;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4j + m passes the
// address of 4 consecutive bf16 of row j, and lane i receives column i of the
// four rows.  Two such reads give one lane 8 consecutive rows of its column:
// the MFMA operand layout of a k-major (transposed) view of a row-major tile.
__device__ __forceinline__ s16x4 ds_read_tr16(const uint16_t* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(lds_ptr));
}

// Operand fragment of lane (l = 16 g + 4 j + m) holding column c0 + 16 (g & 1)
// + (l & 15) and rows r0 + 4 (g >> 1) + t, t = 0..3 then r0 + 8 + 4 (g >> 1) + t,
// t = 0..3 (physical LDS rows), from a SwzTile<D>.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int lane, int r0, int c0) {
  const int g = lane >> 4, j = (lane >> 2) & 3, m = lane & 3;
  const int row = r0 + 4 * (g >> 1) + j;
  const int col = c0 + 16 * (g & 1) + 4 * m;
  const s16x4 lo = ds_read_tr16(tile + SwzTile<D>::elem(row, col));
  const s16x4 hi = ds_read_tr16(tile + SwzTile<D>::elem(row + 8, col));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Byte address of an LDS object (the 32-bit LDS address space).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// Direct global -> LDS copy of 16 bytes per lane: lane i reads sbase + voff
// (sbase wave-uniform, voff its own byte offset) and its bytes land at LDS
// byte address lds + 16 i (lds wave-uniform).  The copy is issued from inline
// assembly so that the compiler does not track its LDS write: it cannot tell
// the buffers of a multi-buffered tile apart and would otherwise make every
// transpose read wait for all copies in flight, which serialises the prefetch
// of the next tile with the current one.  Callers order the copy against
// reads of its destination themselves (s_waitcnt on vmcnt followed by a
// workgroup barrier before the first read).
__device__ __forceinline__ void load_lds16(const void* sbase, uint32_t voff, uint32_t lds) {
  // both bases are wave-uniform; readfirstlane keeps them in scalar registers
  // even where the compiler cannot prove it
  // (readfirstlane returns int: each half goes back through uint32_t so the
  // low half is zero-extended, not sign-extended, into the 64-bit address)
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))));
  sbase = reinterpret_cast<const void*>(uint64_t(lo) | (uint64_t(hi) << 32));
  const uint32_t m0 = uint32_t(__builtin_amdgcn_readfirstlane(int(lds)));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// N direct loads of 16 bytes per lane into N consecutive 1 KB LDS blocks
// ending at byte address lds_top (wave-uniform): load u lands at lds_top -
// 1024 (N - 1 - u) + 16 lane and reads sbase + voff[u] - 1024 (N - 1 - u).
// The hardware adds an instruction's immediate offset to both its global and
// its LDS address, so one M0 value serves all N loads; callers raise voff[u]
// by 1024 (N - 1 - u) to read where they mean.
template <int N>
__device__ __forceinline__ void load_lds16_group(const void* sbase, const uint32_t (&voff)[N],
                                                 uint32_t lds_top) {
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))));
  sbase = reinterpret_cast<const void*>(uint64_t(lo) | (uint64_t(hi) << 32));
  const uint32_t m0 = uint32_t(__builtin_amdgcn_readfirstlane(int(lds_top)));
  static_assert(N == 2 || N == 4, "grouped direct loads come in twos or fours");
  if constexpr (N == 2)
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %2 offset:-1024\n\t"
                 "global_load_lds_dwordx4 %1, %2"
                 :
                 : "v"(voff[0]), "v"(voff[1]), "s"(sbase), "s"(m0)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %5\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %4 offset:-3072\n\t"
                 "global_load_lds_dwordx4 %1, %4 offset:-2048\n\t"
                 "global_load_lds_dwordx4 %2, %4 offset:-1024\n\t"
                 "global_load_lds_dwordx4 %3, %4"
                 :
                 : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}

// The direct loads of a pair of ROWS x D bf16 tiles (the same rows of two
// [T, H, D] tensors) into SwzTile layout, spread over the NW waves of a
// workgroup.  Load u of a lane fills one LDS block (1 KB: 64 lanes x 16
// bytes): block wave N + u when every wave has the same number N > 1 of
// loads (so a wave's loads of one tensor share one M0 value), else u NW +
// wave; the lane that lands on LDS row p, chunk pc fetches source row
// swap_bits23(p), chunk pc ^ swz(p).  The lane's byte offsets relative to the
// tile's first row are computed once, so a tile costs one scalar base
// pointer per tensor.  Near the end of a document, rows at or past n_valid
// are clamped to its last row (whose values are then masked wherever used).
template <int D, int ROWS, int NW>
struct PairLoader {
  static constexpr int NCH = D / 8;            // 16-byte chunks per row
  static constexpr int RPL = 64 / NCH;         // rows per 1 KB block
  static constexpr int BLKS = ROWS / RPL;
  static constexpr int N = (BLKS + NW - 1) / NW;   // loads per lane per tensor
  static constexpr bool kGrouped = N > 1 && BLKS == N * NW;
  uint32_t voff[N];

  __device__ __forceinline__ static int block(int u, int wave) {
    return kGrouped ? wave * N + u : u * NW + wave;
  }

  // wave-uniform: whether load u of this wave exists
  __device__ __forceinline__ static bool has(int u, int wave) {
    return BLKS % NW == 0 || u * NW + wave < BLKS;
  }

  __device__ __forceinline__ static int src_row(int u, int wave, int lane) {
    return swap_bits23(block(u, wave) * RPL + lane / NCH);
  }
  __device__ __forceinline__ static uint32_t col_bytes(int u, int wave, int lane) {
    const int p = block(u, wave) * RPL + lane / NCH;
    return uint32_t(((lane % NCH) ^ SwzTile<D>::swz(p)) << 4);
  }
  __device__ __forceinline__ PairLoader(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int u = 0; u < N; ++u)
      voff[u] = uint32_t(src_row(u, wave, lane)) * row_bytes + col_bytes(u, wave, lane) +
                (kGrouped ? uint32_t(1024 * (N - 1 - u)) : 0u);
  }
  // a, b: first row of the tile in each tensor (wave-uniform)
  __device__ __forceinline__ void issue(const uint16_t* a, const uint16_t* b, uint32_t da,
                                        uint32_t db, int wave) const {
    if constexpr (kGrouped) {
      const uint32_t top = uint32_t((wave * N + N - 1) * 1024);
      load_lds16_group<N>(a, voff, da + top);
      load_lds16_group<N>(b, voff, db + top);
    } else {
#pragma unroll
      for (int u = 0; u < N; ++u) {
        if (!has(u, wave)) continue;
        load_lds16(a, voff[u], da + block(u, wave) * 1024);
        load_lds16(b, voff[u], db + block(u, wave) * 1024);
      }
    }
  }
  __device__ __forceinline__ void issue_clamped(const uint16_t* a, const uint16_t* b, uint32_t da,
                                                uint32_t db, int wave, int lane, int n_valid,
                                                uint32_t row_bytes) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      if (!has(u, wave)) continue;
      const uint32_t o = uint32_t(min(src_row(u, wave, lane), n_valid - 1)) * row_bytes +
                         col_bytes(u, wave, lane);
      load_lds16(a, o, da + block(u, wave) * 1024);
      load_lds16(b, o, db + block(u, wave) * 1024);
    }
  }
  // a tile whose first rows are at a, b, with n_left rows of the document
  // from there on
  __device__ __forceinline__ void load_from(const uint16_t* a, const uint16_t* b, int n_left,
                                            uint32_t row_bytes, uint32_t da, uint32_t db,
                                            int wave, int lane) const {
    if (n_left >= ROWS)
      issue(a, b, da, db, wave);
    else
      issue_clamped(a, b, da, db, wave, lane, n_left, row_bytes);
  }
  // tile of rows row0 .. row0 + ROWS - 1 of a document with n_rows rows;
  // a, b point at the document's first row
  __device__ __forceinline__ void load(const uint16_t* a, const uint16_t* b, int64_t row_elems,
                                       int row0, int n_rows, uint32_t da, uint32_t db, int wave,
                                       int lane) const {
    const int64_t o = int64_t(row0) * row_elems;
    if (row0 + ROWS <= n_rows)
      issue(a + o, b + o, da, db, wave);
    else
      issue_clamped(a + o, b + o, da, db, wave, lane, n_rows - row0, uint32_t(row_elems * 2));
  }
};

// Direct loads of a 128-row x D bf16 tile (rows of one [T, H, D] tensor,
// base = its first row) into two 64-row SwzTile halves at LDS byte addresses
// lo (rows 0-63) and hi (rows 64-127), spread over 4 waves: lane i of 1 KB
// block j fills local row j * RPL + i / NCH.  Rows at or past n_valid (>= 1)
// repeat row n_valid - 1.
template <int D>
__device__ __forceinline__ void load_rows128_lds(const uint16_t* base, uint32_t row_bytes,
                                                 int n_valid, uint32_t lo, uint32_t hi, int wave,
                                                 int lane) {
  constexpr int NCH = D / 8;            // 16-byte chunks per row
  constexpr int RPL = 64 / NCH;         // rows per 1 KB block
  constexpr int NBLK = 128 / RPL;       // blocks of the tile
#pragma unroll
  for (int u = 0; u < NBLK / 4; ++u) {
    const int j = u * 4 + wave;
    const int row = j * RPL + lane / NCH;
    const int p = row & 63;
    const uint32_t pc = uint32_t((lane % NCH) ^ SwzTile<D>::swz(p));
    const uint32_t off = uint32_t(min(row, n_valid - 1)) * row_bytes + (pc << 4);
    load_lds16(base, off, (row < 64 ? lo : hi) + uint32_t((j % (64 / RPL)) * 1024));
  }
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// in 6:4, lgkmcnt in 11:8)
constexpr int kWaitAll = 0;           // every counter at zero
constexpr int kWaitLgkm = 0xC07F;     // LDS / scalar memory only; loads in flight may stay

// integral constant for compile-time buffer indices
template <int V>
struct IC {
  static constexpr int value = V;
};

// Exchange a value with the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// max / sum of x over lanes l and l ^ 32, on the VALU (v_permlane32_swap):
// the swap leaves x of lane l % 32 in one result and x of lane 32 + l % 32 in
// the other, in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace vl
