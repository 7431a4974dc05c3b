// Device helpers shared by the gfx950 attention kernels: operand types, the
// 32x32x16 MFMA wrappers, fp32 -> fp16/bf16 packing, the LDS tile layouts
// with their HBM -> LDS copies and operand reads.
//
// Register layouts of v_mfma_f32_32x32x16_{f16,bf16} (one wave, lane i):
//   A (32 x 16, M x K): lane i holds A[i % 32][8*(i/32) + 0..7]
//   B (16 x 32, K x N): lane i holds B[8*(i/32) + 0..7][i % 32]
//   C (32 x 32)       : lane i, register r holds C[row(i, r)][i % 32] with
//                       row(i, r) = 8*(r/4) + 4*(i/32) + r%4
// Only the pairing of A's and B's k-slots matters for a contraction, so a
// kernel may feed any consistent permutation of the k index to both.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

enum { DT_F16 = 0, DT_BF16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);

template <>
__device__ __forceinline__ f32x16 mfma32<DT_F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<DT_BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Two fp32 values rounded to nearest-even into one dword (lo in bits 0..15).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<DT_F16>(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<DT_BF16>(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Row of the 32x32 accumulator held by lane-half `half` in register r.
__device__ __forceinline__ int acc_row(int half, int r) { return ((r >> 2) << 3) + (half << 2) + (r & 3); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane l receives element
// j (j = 0..3) from the 8-byte word addressed by lane 4*j + (l%16)/4 of the
// group, at 16-bit offset l%4.  With lane p of a group pointing at
// (row0 + p/4, col0 + 4*(p%4)), lane l gets rows row0..row0+3 of column
// col0 + l%16: a 4-key x 16-column transpose.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds_ptr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// ---------------------------------------------------------------- LDS tiles
//
// A tile holds 32 rows (keys or queries) of D 16-bit elements.  It is filled
// by HBM -> LDS copies of 1 KiB per wave instruction (lane i writes bytes
// 16 i .. 16 i + 15 of the instruction's block; buffer_load ... lds, no
// staging registers) and read as MFMA operands in two patterns:
//
//   row-major operand, k over the d columns: lane i reads the 8 columns
//     16 ks + 8 (i/32) .. +7 of row i % 32 (one ds_read_b128 per k step ks);
//   transposed operand, k over the rows, m over the d columns: lane i gets
//     column 32 db + i%32 of rows {16 kk + 4 (i/32) + 0..3, +8 + 0..3},
//     matching the k order of a 32x32 accumulator's registers 8 kk .. 8 kk+7
//     (see acc_row), from two ds_read_b64_tr_b16 whose 16-lane groups each
//     cover 4 rows x 16 columns.
//
// Each layout makes both read patterns free of LDS bank conflicts and lets
// every group of four lanes of a copy instruction fetch 64 contiguous bytes
// of one row.  TileLayout<D> holds a lane's read offsets; rm_off(ks) and
// tr_off(kk, db, hi) are byte offsets from the tile's base (hi: rows +8).

template <int D>
struct TileLayout;

// d = 64: rows of 128 bytes (8 chunks of 16 bytes); chunk c of row r lives
// at physical chunk c ^ swz(r).  The XOR spreads 16 consecutive rows of one
// chunk and 4 rows x 4 chunks over distinct banks; the k-step offsets of a
// lane are not affine, so they are kept per lane (6 registers).
template <>
struct TileLayout<64> {
  static constexpr int D = 64;
  static constexpr int BYTES = 32 * D * 2;
  static __device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
  static __device__ __forceinline__ int elem_off(int r, int col) {
    return r * D + ((((col >> 3) ^ swz(r)) << 3) | (col & 7));
  }
  uint32_t rm[D / 16];
  uint32_t tr[D / 32][2];

  __device__ __forceinline__ void init(int lane) {
    const int col = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) rm[ks] = 2u * (uint32_t)(col * D + (((2 * ks + half) ^ swz(col)) << 3));
    const int g = lane >> 4, p = lane & 15;
    const int row0 = 4 * (g >> 1) + (p >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int c = db * 32 + 16 * (g & 1) + 4 * (p & 3);
      tr[db][0] = 2u * (uint32_t)elem_off(row0, c);
      tr[db][1] = 2u * (uint32_t)elem_off(row0 + 8, c);
    }
  }
  __device__ __forceinline__ uint32_t rm_off(int ks) const { return rm[ks]; }
  // the swizzle repeats every 16 rows, so the k block is a plain row offset
  __device__ __forceinline__ uint32_t tr_off(int kk, int db, int hi) const { return tr[db][hi] + kk * 16u * D * 2u; }

  // Copy rows [0, 32) of one head's [N][64] tensor (row stride row_bytes,
  // first row at byte tile_byte_off) into the tile at `lds`, spread over
  // WAVES waves: lane i of an instruction fetches the global chunk whose
  // swizzled home is byte 16 i of the instruction's block of 8 rows.
  template <int WAVES>
  static __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, uint32_t tile_byte_off,
                                               uint16_t* lds, int lane, int wave) {
    constexpr int NI = 4 / WAVES;
    static_assert(NI >= 1 && NI * WAVES == 4, "tile must split evenly over the waves");
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = (wave * NI + i) * 8 + lane / 8;
      const int c = (lane % 8) ^ swz(r);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + (wave * NI + i) * 8 * D), 16,
          (uint32_t)r * row_bytes + (uint32_t)(c * 16), tile_byte_off, 0, 0);
    }
  }
  template <int WAVES>
  static constexpr int copy_insts() { return 4 / WAVES; }
};

// d = 128: 8 blocks of 4 rows, each block 1 KiB of data plus 16 bytes of
// padding (stride 1040).  Inside a block, chunk c (16 bytes) of row t sits
// at position 16 (c / 4) + 4 t + c % 4.  So a copy instruction fills one
// block from 4 consecutive rows, each group of four lanes fetching 64
// contiguous bytes, and the address of (row r, chunk c) splits into a row
// part and a chunk part: every read of a tile is one per-lane base plus
// immediate offsets (no per-k-step address registers or adds).  The
// 16-byte shift per block plus the 4 t term put 16 consecutive rows of one
// chunk, and 4 rows x 4 consecutive chunks, on distinct banks.
template <>
struct TileLayout<128> {
  static constexpr int BLK = 1040;
  static constexpr int BYTES = 8 * BLK;
  uint32_t rb, tb;  // lane bases of the row-major and transposed reads

  __device__ __forceinline__ void init(int lane) {
    const int r = lane & 31, h = lane >> 5;
    rb = (uint32_t)((r >> 2) * BLK + (4 * (r & 3) + h) * 16);
    const int g = lane >> 4, p = lane & 15;
    tb = (uint32_t)((g >> 1) * BLK + (4 * (p >> 2) + 2 * (g & 1) + ((p >> 1) & 1)) * 16 + (p & 1) * 8);
  }
  __device__ __forceinline__ uint32_t rm_off(int ks) const { return rb + 256u * (ks >> 1) + 32u * (ks & 1); }
  __device__ __forceinline__ uint32_t tr_off(int kk, int db, int hi) const {
    return tb + (uint32_t)(kk * 4 * BLK + db * 256 + hi * 2 * BLK);
  }

  // Copy rows [0, 32) of one head's [N][128] tensor (row stride row_bytes,
  // first row at byte tile_byte_off) into the tile at `lds`, one block per
  // instruction, spread over WAVES waves.
  template <int WAVES>
  static __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, uint32_t row_bytes, uint32_t tile_byte_off,
                                               uint16_t* lds, int lane, int wave) {
    constexpr int NI = 8 / WAVES;
    static_assert(NI >= 1 && NI * WAVES == 8, "tile must split evenly over the waves");
    const int t = (lane >> 2) & 3, c = 4 * (lane >> 4) + (lane & 3);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int b = wave * NI + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)((char*)lds + b * BLK), 16,
          (uint32_t)(4 * b + t) * row_bytes + (uint32_t)(c * 16), tile_byte_off, 0, 0);
    }
  }
  template <int WAVES>
  static constexpr int copy_insts() { return 8 / WAVES; }
};

// Elements of one 32-row tile slot (16-bit units), for sizing LDS rings.
template <int D>
constexpr int kTileElems = TileLayout<D>::BYTES / 2;

__device__ __forceinline__ u32x4 lds_b128(const uint16_t* base, uint32_t byte_off) {
  return *(const u32x4*)((const char*)base + byte_off);
}
// Row-major operand of k step ks.
template <int D>
__device__ __forceinline__ u32x4 lds_rowmajor(const uint16_t* base, const TileLayout<D>& ta, int ks) {
  return lds_b128(base, ta.rm_off(ks));
}
// Transposed operand of k block kk (rows 16 kk ..) and d block db.
template <int D>
__device__ __forceinline__ u32x4 lds_transposed_a(const uint16_t* base, const TileLayout<D>& ta, int kk, int db) {
  const char* b = (const char*)base;
  u32x2 lo = lds_read_tr16((const uint16_t*)(b + ta.tr_off(kk, db, 0)));
  u32x2 hi = lds_read_tr16((const uint16_t*)(b + ta.tr_off(kk, db, 1)));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Pin the issue order of a straight-line run of NM MFMAs fed by NR LDS
// reads: the reads of the first kReadLead MFMAs go first, then each MFMA
// is followed by an even share of the remaining reads, so an operand is
// read about kReadLead MFMAs (kReadLead x 32 cycles) before its use and the
// LDS latency hides under the matrix core.  Without this the scheduler
// issues each read right before its MFMA.
constexpr int kReadLead = 4;
template <int NM, int NR>
__device__ __forceinline__ void sched_reads_ahead() {
  if constexpr (NM <= kReadLead) {  // a short run: every read first
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  } else {
    constexpr int first = NR * kReadLead / NM;
    constexpr int rest = NR - first;
    constexpr int per = (rest + NM - kReadLead - 1) / (NM - kReadLead);
    __builtin_amdgcn_sched_group_barrier(0x100, first, 0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NM - kReadLead) __builtin_amdgcn_sched_group_barrier(0x100, per, 0);
    }
  }
}

// Pack registers 8*kk .. 8*kk+7 of an fp32 accumulator into an MFMA operand.
template <int DT>
__device__ __forceinline__ u32x4 pack_acc8(const f32x16& s, int kk) {
  const int o = 8 * kk;
  return u32x4{pack2<DT>(s[o + 0], s[o + 1]), pack2<DT>(s[o + 2], s[o + 3]), pack2<DT>(s[o + 4], s[o + 5]),
               pack2<DT>(s[o + 6], s[o + 7])};
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64-bit products and
// xors, the key bumped by the two Weyl constants between rounds.  Dropout
// draws one call per (query row, 16 keys of a 32-key tile).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t a = (uint64_t)0xD2511F53u * c0;
    const uint64_t b = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(b >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(a >> 32) ^ c3 ^ k1;
    c0 = n0;
    c1 = (uint32_t)b;
    c2 = n2;
    c3 = (uint32_t)a;
  }
  return u32x4{c0, c1, c2, c3};
}

// Combine lane i with lane i^32.  (v_permlane32_swap would avoid the LDS
// round trip of ds_bpermute, but this compiler maps the builtin's second
// result onto the first one's register, so it cannot be used for this.)
__device__ __forceinline__ float max_pair32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float sum_pair32(float x) { return x + __shfl_xor(x, 32); }

// ---------------------------------------------------------------- HBM -> LDS

// Buffer resource over one head's rows of a [N][d] 16-bit tensor with row
// stride `stride` elements: loads past row n-1 return zeros.  The byte
// count is unsigned: the host admits per-head extents of up to 2^31 - 1
// elements, i.e. up to 2^32 - 2 bytes, which the 32-bit field holds.
__device__ __forceinline__ uint32_t rsrc_bytes(int64_t bytes) { return (uint32_t)bytes; }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int n, int64_t stride, int d) {
  const uint32_t bytes = rsrc_bytes(((int64_t)(n - 1) * stride + d) * 2);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, __builtin_bit_cast(int, bytes), 0x00020000);
}
// Buffer resource over n fp32 values (zeros past the end).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t f32_rsrc(const float* base, int n) {
  const uint32_t bytes = rsrc_bytes((int64_t)n * 4);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, __builtin_bit_cast(int, bytes), 0x00020000);
}

// Asynchronous copy of N fp32 values (N a multiple of 4, at most 256) into
// LDS by one wave; lanes past N/4 are idle.
template <int N>
__device__ __forceinline__ void vec_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t byte_off, float* lds, int lane) {
  static_assert(N % 4 == 0 && N <= 256, "vector copy size");
  if (lane < N / 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16, lane * 16, byte_off,
                                             0, 0);
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// vmcnt(n): wait until at most n vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those make every wave wait for all of its outstanding HBM->LDS copies,
// including the prefetch that should stay in flight.  Ordering of the LDS
// rings comes from the explicit vmcnt waits before it; the empty asm
// statements keep the compiler from moving memory accesses across it.
// The wave's own LDS reads must also be complete (lgkmcnt 0) when it
// arrives: the compiler may place the MFMAs that consume the last reads
// after the barrier, and their lgkmcnt waits with them, while the copies
// issued after the barrier may refill the slot those reads come from.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace fa
