// Device helpers shared by the MXFP8 GEMM kernels for gfx950 (internal).
//
// Hardware mapping (measured on the device):
//   v_mfma_scale_f32_32x32x64_f8f6f4, wave64.  Operand lane l holds row l%32;
//   lane half g = l/32 holds K bytes [16g, 16g+16) of scale block 0 and
//   [32+16g, 32+16g+16) of scale block 1; the scale of block b for row i is
//   the byte (op_sel) of lane i + 32b's scale register.  Result lane l, acc
//   j: row 8(j/4) + 4(l/32) + j%4, column l%32.
// The MFMA's first operand is B (the N side) and its second is A (the M
// side), so each lane ends with groups of four consecutive n of one C row;
// lanes l and l + 32 trade groups (v_permlane32_swap) so that every store
// writes 8 consecutive BF16 (16 bytes).
#pragma once
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int NT = 256;
constexpr int A_TILE = BM * BK;           // 32 KB
constexpr int B_TILE = BN * BK;           // 32 KB
constexpr int STAGE = A_TILE + B_TILE;    // 64 KB
constexpr int SCALE_TILE = 2 * 256 * 16; // A and B scale bytes of four K steps: 8 KB
constexpr int PF_DIST = 3;                // L2 prefetch distance, in K steps
constexpr int GM_TILES = 8;               // tile grouping along M (tile_of)
constexpr int CHUNKS = A_TILE / 16 / NT;  // 16-byte chunks per thread per operand: 8
constexpr int MAX_GROUPS = 512;

// Row-major LDS tiles with 128-byte rows keep 16-byte chunk c of row r at
// physical chunk c ^ ((r >> 1) & 7).  gfx950 LDS serves 256 bytes (64
// banks) per cycle, i.e. 16 lanes of a 16-byte read; the 16 lanes of a
// fragment read take rows r .. r+15 at one logical chunk, and this swizzle
// puts them in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// Fragment of 32 rows x 64 K from a row-major LDS tile (128-byte rows).
__device__ __forceinline__ v8i read_frag(const lds_u8* tile, int row, int s, int g) {
  const int x = swz(row);
  v4i lo = *(const lds_v4i*)(tile + row * BK + (((2 * s + g) ^ x) << 4));
  v4i hi = *(const lds_v4i*)(tile + row * BK + (((4 + 2 * s + g) ^ x) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Fragment of 32 columns x 64 K from a [128 k][256 n] LDS tile (256-byte
// rows), read transposed with ds_read_b64_tr_b8: in each group of 16 lanes,
// lane 2r+h points at 8 bytes of row k+r and lane i receives byte i of the
// eight 16-byte rows, i.e. 8 consecutive k of column i.
__device__ __forceinline__ v8i read_frag_t(const lds_u8* tile, int nb, int s, int lane) {
  const int g = lane >> 5, q = (lane >> 4) & 1, r = (lane & 15) >> 1, hh = lane & 1;
  // row k = k_const + 16g + r with k_const a multiple of 8, so k & 7 = r and
  // the swizzled chunk is lane-only; every piece is base + a constant offset.
  // Chunk c of row k sits at physical chunk c ^ 2(k & 7): the two 16-lane
  // groups served together read chunks c, c+1 (c even) of the same 8 rows,
  // which land on 16 distinct 16-byte bank groups.
  const int ncol = nb + 16 * q + 8 * hh;
  const lds_u8* base = tile + (16 * g + r) * 256 + (((ncol >> 4) ^ (2 * r)) << 4) + (ncol & 15);
  v2i p[4];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int kc = (t >> 1) * 64 + 32 * s + (t & 1) * 8;
    p[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(base + kc * 256));
  }
  return (v8i){p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

// Raw buffer descriptor over [base, base + bytes): loads at offsets >= bytes
// return zero, which fills the tile edges (rows past M or N, K past the end).
// Every input is uniform across the wave; readfirstlane makes that visible
// to the compiler so the descriptor lives in scalar registers.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, int64_t bytes) {
  const uint64_t p = (uint64_t)base;
  return (u32x4){(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xFFFFu)),
                 (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bytes), 0x00020000u};
}

// 16 bytes per lane from the buffer at voffset into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds).  Issued through asm so that the compiler does
// not order LDS reads of the other stage behind these loads; the kernel waits
// for them itself (vmcnt(0) before the barrier that publishes the stage).
__device__ __forceinline__ void dma16(const lds_u8* lds, uint32_t voffset, u32x4 rsrc) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory");
}

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima), as a builtin so
// the compiler knows every earlier vector-memory load has completed.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(2): everything but the two most recent vector-memory ops
// (the L2 prefetches, which nobody waits for) has completed.
__device__ __forceinline__ void wait_vm_but_prefetch() { __builtin_amdgcn_s_waitcnt(0x0F72); }

// s_waitcnt vmcnt(N) for any N < 64 (gfx9 encoding: the count's low four
// bits in [3:0], its high two in [15:14]; expcnt and lgkmcnt at their maxima).
// Vector-memory loads and stores retire in order, so this waits for every
// vector-memory op but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// L2 prefetch: one dword per lane (one 128-byte line per row) dropped into a
// scratch LDS area that is never read.  LDS-DMA has no register destination,
// so nothing in the kernel can race with the late arrival.
__device__ __forceinline__ void prefetch_lines(const lds_u8* scratch, uint32_t voffset, u32x4 rsrc) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)scratch);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory");
}

constexpr uint32_t OOB = 0x80000000u;  // an offset past every tile buffer

// 4 bytes per lane from the buffer at voffset into LDS at lds + 4 * lane
// (buffer_load_dword ... lds), waited for like dma16.
__device__ __forceinline__ void dma4(const lds_u8* lds, uint32_t voffset, u32x4 rsrc) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory");
}

// The 16 MFMAs of one 64-K half (S = 0, 1) of a K step for a wave's 128x128
// sub-tile: B fragments are the first operand, A fragments the second, and
// op_sel S picks byte S of each lane's scale word.  FA / FB are the element
// formats of A and B in the MFMA's encoding (0 = E4M3, 1 = E5M2), passed as
// the formats of the instruction's first (B) and second (A) operand.
template <int S, int FA = 0, int FB = 0>
__device__ __forceinline__ void mma_tile(const v8i* af, const v8i* bf, const uint32_t* sar,
                                         const uint32_t* sbr, v16f (&acc)[4][4]) {
#pragma unroll
  for (int fn = 0; fn < 4; fn++)
#pragma unroll
    for (int fm = 0; fm < 4; fm++)
      acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          bf[fn], af[fm], acc[fn][fm], FB, FA, S, (int)sbr[fn], S, (int)sar[fm]);
}

// Ask the scheduler for MFMA, LDS read, vector load, MFMA, ... so the MFMA
// pipe always has queued work while the loads are in flight.
template <int NDS, int NVM>
__device__ __forceinline__ void interleave_ops() {
  constexpr int ds_per = (NDS + 15) / 16, vm_per = (NVM + 15) / 16;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // MFMA
    if (ds_per) __builtin_amdgcn_sched_group_barrier(0x100, ds_per, 0);  // DS read
    if (vm_per) __builtin_amdgcn_sched_group_barrier(0x020, vm_per, 0);  // VMEM read
  }
}

// Epilogue of a 256x256 tile: FP32 -> BF16 (RNE) into C (row stride ldc).
// A lane holds four consecutive n of its row per group r4 (n = 8 r4 + 4 g +
// 0..3); one v_permlane32_swap per dword pair trades groups between lanes l
// and l + 32, after which lane half g holds the 8 consecutive n at 8 g + 16 h
// for h = 0, 1 and stores them as one 16-byte write.  The swaps run on every
// lane before any lane drops out at the M edge.
__device__ __forceinline__ void store_tile_bf16(const v16f (&acc)[4][4], uint16_t* __restrict__ c,
                                                int64_t ldc, int64_t m0, int64_t m_end, int64_t n0,
                                                int64_t N, int wm, int wn, int lane) {
  const int g = lane >> 5, i = lane & 31;
  const bool vec_ok = (ldc & 7) == 0;
#pragma unroll
  for (int fn = 0; fn < 4; fn++) {
#pragma unroll
    for (int fm = 0; fm < 4; fm++) {
      const v16f& v = acc[fn][fm];
      uint32_t p[4][2];
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        p[r4][0] = cvt_pk_bf16(v[4 * r4 + 0], v[4 * r4 + 1]);
        p[r4][1] = cvt_pk_bf16(v[4 * r4 + 2], v[4 * r4 + 3]);
      }
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int d = 0; d < 2; d++) {
          const auto s = __builtin_amdgcn_permlane32_swap(p[2 * h][d], p[2 * h + 1][d], false, false);
          p[2 * h][d] = s[0];
          p[2 * h + 1][d] = s[1];
        }
      const int64_t m = m0 + 128 * wm + 32 * fm + i;
      if (m >= m_end) continue;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int64_t n = n0 + 128 * wn + 32 * fn + 16 * h + 8 * g;
        const uint32_t w[4] = {p[2 * h][0], p[2 * h][1], p[2 * h + 1][0], p[2 * h + 1][1]};
        uint16_t* dst = c + m * ldc + n;
        if (vec_ok && n + 8 <= N) {
          *(uint4*)dst = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; e++)
            if (n + e < N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

// Epilogue of a 256x256 tile through LDS: the BF16 tile is first written to
// the two (idle) stage buffers as 256 rows of 512 bytes, rows 0..127 in lo
// and 128..255 in hi, 16-byte chunk c of row r at chunk c ^ (r & 31), and
// then stored with each group of 32 lanes writing one whole 512-byte row
// (four full cache lines) per instruction, instead of 32-byte pieces of 32
// rows.  The caller has made every load of the stage buffers land and every
// wave pass a barrier since its last read of them.  Ends with a barrier
// (the stage buffers are free again afterwards).
__device__ __forceinline__ void store_tile_bf16_lds(const v16f (&acc)[4][4], lds_u8* lo, lds_u8* hi,
                                                    uint16_t* __restrict__ c, int64_t ldc, int64_t m0,
                                                    int64_t m_end, int64_t n0, int64_t N, int wm,
                                                    int wn, int wave, int lane) {
  const int g = lane >> 5, i = lane & 31;
  lds_u8* buf = wm ? hi : lo;
#pragma unroll
  for (int fn = 0; fn < 4; fn++) {
#pragma unroll
    for (int fm = 0; fm < 4; fm++) {
      const v16f& v = acc[fn][fm];
      uint32_t p[4][2];
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        p[r4][0] = cvt_pk_bf16(v[4 * r4 + 0], v[4 * r4 + 1]);
        p[r4][1] = cvt_pk_bf16(v[4 * r4 + 2], v[4 * r4 + 3]);
      }
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int d = 0; d < 2; d++) {
          const auto sw = __builtin_amdgcn_permlane32_swap(p[2 * h][d], p[2 * h + 1][d], false, false);
          p[2 * h][d] = sw[0];
          p[2 * h + 1][d] = sw[1];
        }
      // local row 32 fm + i of this wave's half; chunk (8 columns) 16 wn + 4 fn + 2 h + g
      const int row = 32 * fm + i;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int chunk = 16 * wn + 4 * fn + 2 * h + g;
        *(lds_v4i*)(buf + row * 512 + ((chunk ^ (row & 31)) << 4)) =
            (v4i){(int)p[2 * h][0], (int)p[2 * h][1], (int)p[2 * h + 1][0], (int)p[2 * h + 1][1]};
      }
    }
  }
  __syncthreads();
  // wave w stores rows 64 w .. 64 w + 63, two rows per instruction: lane l
  // takes chunk l & 31 of row 64 w + 2 j + (l >> 5)
  const int k = lane & 31;
  const int64_t n = n0 + 8 * k;
  if (((ldc | N) & 7) == 0 && (int64_t)BM * ldc * 2 < (int64_t)OOB) {
    // Rows 16-byte aligned and whole 8-column chunks: eight LDS reads, then
    // eight buffer stores, with no branches; rows past m_end and chunks past
    // N get an offset past the descriptor's range and store nothing.  (One
    // read, wait and store per row costs an LDS round trip per row.)
    const int64_t mrows = m_end - m0;
    const uint64_t base = (uint64_t)(uintptr_t)(c + m0 * ldc);
    const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(uintptr_t)(((uint64_t)bhi << 32) | blo), 0,
        __builtin_amdgcn_readfirstlane((int)(mrows * ldc * 2)), 0x00020000);
    // row r = r0 + 2 j of this lane: byte offset off0 + j * step2, stored
    // while 2 j < lim.  off0 is made opaque so that nothing derived from it
    // is hoisted out of a caller's loop over tiles (32 row offsets held
    // across the K loop would spill).
    const int r0 = 64 * wave + (lane >> 5);
    uint32_t row2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(ldc * 2));
    uint32_t off0 = (uint32_t)r0 * row2 + (uint32_t)(8 * k) * 2 + (uint32_t)__builtin_amdgcn_readfirstlane((int)(n0 * 2));
    int lim = n < N ? (int)mrows - r0 : 0;
    asm volatile("" : "+s"(row2), "+v"(off0), "+v"(lim));
    const uint32_t step2 = 2 * row2;
#pragma unroll
    for (int jb = 0; jb < 32; jb += 8) {
      v4i w[8];
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int r = r0 + 2 * (jb + u);
        w[u] = *(const lds_v4i*)((r < 128 ? lo : hi) + (r & 127) * 512 + ((k ^ (r & 31)) << 4));
      }
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const int j = jb + u;
        const uint32_t off = 2 * j < lim ? off0 + (uint32_t)j * step2 : OOB;
        __builtin_amdgcn_raw_buffer_store_b128(w[u], rc, (int)off, 0, 0);
      }
    }
    __syncthreads();
    return;
  }
  const bool vec_ok = (ldc & 7) == 0;
#pragma unroll 4
  for (int j = 0; j < 32; j++) {
    const int r = 64 * wave + 2 * j + (lane >> 5);  // tile row
    const lds_u8* src = (r < 128 ? lo : hi) + (r & 127) * 512 + ((k ^ (r & 31)) << 4);
    const v4i w = *(const lds_v4i*)src;
    const int64_t m = m0 + r;
    if (m >= m_end || n >= N) continue;
    uint16_t* dst = c + m * ldc + n;
    if (vec_ok && n + 8 <= N) {
      *(uint4*)dst = make_uint4((uint32_t)w.x, (uint32_t)w.y, (uint32_t)w.z, (uint32_t)w.w);
    } else {
      const uint32_t ww[4] = {(uint32_t)w.x, (uint32_t)w.y, (uint32_t)w.z, (uint32_t)w.w};
#pragma unroll
      for (int e = 0; e < 8; e++)
        if (n + e < N) dst[e] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
    }
  }
  __syncthreads();
}

// The tile's BF16 result through ONE 64 KB LDS buffer, half at a time, so
// that the other stage buffer can take the next tile's first loads while the
// result leaves.  Half h holds fragment rows fm = 2h, 2h + 1 of every wave,
// i.e. tile rows 128 wm + 64 h .. + 63 for wm = 0, 1 (all four waves convert
// in both halves); its local row lr is tile row 128 (lr / 64) + 64 h +
// lr % 64.  Every wave issues exactly 32 buffer stores, none skipped (rows
// past m_end and chunks past N take an offset past the descriptor's range),
// so a caller can count them in vmcnt.  Requires ldc % 8 == 0, N % 8 == 0
// and 256 * ldc * 2 < 2^31 (the caller checks).  Ends with a barrier.
__device__ __forceinline__ void store_tile_bf16_lds_halves(const v16f (&acc)[4][4], lds_u8* buf,
                                                           uint16_t* __restrict__ c, int64_t ldc,
                                                           int64_t m0, int64_t m_end, int64_t n0,
                                                           int64_t N, int wm, int wn, int wave,
                                                           int lane) {
  const int g = lane >> 5, i = lane & 31;
  const int k = lane & 31;
  const int64_t mrows = m_end - m0;
  const uint64_t base = (uint64_t)(uintptr_t)(c + m0 * ldc);
  const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
  const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(uintptr_t)(((uint64_t)bhi << 32) | blo), 0,
      __builtin_amdgcn_readfirstlane((int)(mrows * ldc * 2)), 0x00020000);
  // store j (< 16) of half h: local row lr = 32 wave + 2 j + lane / 32, tile
  // row tr = 128 (wave / 2) + 64 h + (lr % 64); the byte offset is
  // off0 + (64 h + 2 j) row2 and the row is stored while 64 h + 2 j < lim
  const int lr0 = 32 * wave + (lane >> 5);
  const int tr0 = 128 * (wave >> 1) + (lr0 & 63);
  uint32_t row2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)(ldc * 2));
  uint32_t off0 = (uint32_t)tr0 * row2 + (uint32_t)(8 * k) * 2 +
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)(n0 * 2));
  int lim = n0 + 8 * k < N ? (int)mrows - tr0 : 0;
  // opaque: a caller's loop over tiles must not hoist the 32 row offsets
  // derived from these (they would be held across its K loop and spill)
  asm volatile("" : "+s"(row2), "+v"(off0), "+v"(lim));
#pragma unroll
  for (int h = 0; h < 2; h++) {
#pragma unroll
    for (int fn = 0; fn < 4; fn++) {
#pragma unroll
      for (int f2 = 0; f2 < 2; f2++) {
        const v16f& v = acc[fn][2 * h + f2];
        uint32_t p[4][2];
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          p[r4][0] = cvt_pk_bf16(v[4 * r4 + 0], v[4 * r4 + 1]);
          p[r4][1] = cvt_pk_bf16(v[4 * r4 + 2], v[4 * r4 + 3]);
        }
#pragma unroll
        for (int hh = 0; hh < 2; hh++)
#pragma unroll
          for (int d = 0; d < 2; d++) {
            const auto sw = __builtin_amdgcn_permlane32_swap(p[2 * hh][d], p[2 * hh + 1][d], false, false);
            p[2 * hh][d] = sw[0];
            p[2 * hh + 1][d] = sw[1];
          }
        const int row = 64 * wm + 32 * f2 + i;  // local row
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const int chunk = 16 * wn + 4 * fn + 2 * hh + g;
          *(lds_v4i*)(buf + row * 512 + ((chunk ^ (row & 31)) << 4)) =
              (v4i){(int)p[2 * hh][0], (int)p[2 * hh][1], (int)p[2 * hh + 1][0], (int)p[2 * hh + 1][1]};
        }
        // one fragment at a time: reading every fragment's accumulators
        // ahead would hold them all in vector registers
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < 16; jb += 4) {
      v4i w[4];
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int lr = lr0 + 2 * (jb + u);
        w[u] = *(const lds_v4i*)(buf + lr * 512 + ((k ^ (lr & 31)) << 4));
      }
#pragma unroll
      for (int u = 0; u < 4; u++) {
        const int j = jb + u;
        uint32_t off = 64 * h + 2 * j < lim ? off0 + (uint32_t)(64 * h + 2 * j) * row2 : OOB;
        // an opaque offset: the store is issued on every lane, never turned
        // into a masked (possibly skipped) one
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_raw_buffer_store_b128(w[u], rc, (int)off, 0, 0);
      }
    }
    __syncthreads();
  }
}

// Fused producer epilogue: the tile's BF16 result (the same values
// store_tile_bf16 writes) quantised in 1x32 blocks along N, written as
// payload q [M, ldq] (EL: E4M3 or E5M2) and scales s [M, ldq / 32].  After
// the lane-pair swap of store_tile_bf16, lanes i and i + 32 together hold the
// 32 columns of one block (16 each): a block's amax is one exchange between
// them, and the scale and conversion are those of the row quantiser, so the
// bytes equal quantising the BF16 output.  Requires N % 32 == 0.
template <int EL>
__device__ __forceinline__ void store_tile_q(const v16f (&acc)[4][4], uint8_t* __restrict__ q,
                                             uint8_t* __restrict__ s, int64_t ldq, int64_t m0,
                                             int64_t m_end, int64_t n0, int64_t N, int wm, int wn,
                                             int lane) {
  const int g = lane >> 5, i = lane & 31;
#pragma unroll
  for (int fn = 0; fn < 4; fn++) {
#pragma unroll
    for (int fm = 0; fm < 4; fm++) {
      const v16f& v = acc[fn][fm];
      uint32_t p[4][2];
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        p[r4][0] = cvt_pk_bf16(v[4 * r4 + 0], v[4 * r4 + 1]);
        p[r4][1] = cvt_pk_bf16(v[4 * r4 + 2], v[4 * r4 + 3]);
      }
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int d = 0; d < 2; d++) {
          const auto sw = __builtin_amdgcn_permlane32_swap(p[2 * h][d], p[2 * h + 1][d], false, false);
          p[2 * h][d] = sw[0];
          p[2 * h + 1][d] = sw[1];
        }
      // this lane's 16 values: h = 0 -> p[0], p[1]; h = 1 -> p[2], p[3]
      uint32_t m = 0;
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) m = umax(m, umax(pair_absmax(p[r4][0]), pair_absmax(p[r4][1])));
      m = umax(m, (uint32_t)__shfl_xor((int)m, 32, 64));
      const uint32_t sb = scale_byte_t<EL>(m);
      const int64_t row = m0 + 128 * wm + 32 * fm + i;
      const int64_t nb = n0 + 128 * wn + 32 * fn;  // first column of the block
      if (row >= m_end || nb >= N) continue;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const uint4 w = make_uint4(p[2 * h][0], p[2 * h][1], p[2 * h + 1][0], p[2 * h + 1][1]);
        *(uint2*)(q + row * ldq + nb + 16 * h + 8 * g) = cvt8_t<EL>(w, sb);
      }
      if (g == 0) s[row * (ldq >> 5) + (nb >> 5)] = (uint8_t)sb;
    }
  }
}

// The halves epilogue of store_tile_bf16_lds_halves for the fused producer:
// the BF16 rows staged in LDS are quantised in 1x32 blocks on their way out
// (the four lanes holding a block's 16-byte chunks share its amax through a
// quad DPP reduction; the same rounding to BF16 and the same scale rule as
// the row quantiser), payload rows leave whole (8 bytes per lane, 256 bytes
// per row), and each row's 8 scale bytes are gathered in `sst` (2 KB) and
// stored as one 8-byte piece at the end.  Exactly 33 buffer stores per wave
// (32 payload, 1 scale), rows past m_end at an out-of-range offset.
// Requires N % 256 == 0 (whole tiles, 8-byte aligned scale pieces) and
// 256 N < 2^31.
template <int EL, int QR = 2>
__device__ __forceinline__ void store_tile_q_lds_halves(const v16f (&acc)[4][4], lds_u8* buf,
                                                        lds_u8* sst, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ s, int64_t N,
                                                        int64_t m0, int64_t m_end, int64_t n0,
                                                        int wm, int wn, int wave, int lane) {
  const int g = lane >> 5, i = lane & 31;
  const int k = lane & 31;
  const int64_t mrows = m_end - m0;
  const int64_t lds_ = N >> 5;  // scale bytes per row
  const uint64_t qb = (uint64_t)(uintptr_t)(q + m0 * N);
  const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(qb >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)qb)),
      0, __builtin_amdgcn_readfirstlane((int)(mrows * N)), 0x00020000);
  const uint64_t sbase = (uint64_t)(uintptr_t)(s + m0 * lds_);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sbase >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sbase)),
      0, __builtin_amdgcn_readfirstlane((int)(mrows * lds_)), 0x00020000);
  // store j (< 16) of half h: local row lr = 32 wave + 2 j + lane / 32, tile
  // row tr0 + 64 h + 2 j as in the BF16 form; payload byte offset
  // off0 + (64 h + 2 j) N
  const int lr0 = 32 * wave + (lane >> 5);
  const int tr0 = 128 * (wave >> 1) + (lr0 & 63);
  uint32_t rowq = (uint32_t)__builtin_amdgcn_readfirstlane((int)N);
  uint32_t off0 = (uint32_t)tr0 * rowq + (uint32_t)(8 * k) +
                  (uint32_t)__builtin_amdgcn_readfirstlane((int)n0);
  int lim = (int)mrows - tr0;
  // opaque, as in the BF16 form: not hoisted across a caller's K loop
  asm volatile("" : "+s"(rowq), "+v"(off0), "+v"(lim));
#pragma unroll
  for (int h = 0; h < 2; h++) {
#pragma unroll
    for (int fn = 0; fn < 4; fn++) {
#pragma unroll
      for (int f2 = 0; f2 < 2; f2++) {
        const v16f& v = acc[fn][2 * h + f2];
        uint32_t p[4][2];
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          p[r4][0] = cvt_pk_bf16(v[4 * r4 + 0], v[4 * r4 + 1]);
          p[r4][1] = cvt_pk_bf16(v[4 * r4 + 2], v[4 * r4 + 3]);
        }
#pragma unroll
        for (int hh = 0; hh < 2; hh++)
#pragma unroll
          for (int d = 0; d < 2; d++) {
            const auto sw = __builtin_amdgcn_permlane32_swap(p[2 * hh][d], p[2 * hh + 1][d], false, false);
            p[2 * hh][d] = sw[0];
            p[2 * hh + 1][d] = sw[1];
          }
        const int row = 64 * wm + 32 * f2 + i;  // local row
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const int chunk = 16 * wn + 4 * fn + 2 * hh + g;
          *(lds_v4i*)(buf + row * 512 + ((chunk ^ (row & 31)) << 4)) =
              (v4i){(int)p[2 * hh][0], (int)p[2 * hh][1], (int)p[2 * hh + 1][0], (int)p[2 * hh + 1][1]};
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int jb = 0; jb < 16; jb += QR) {
      v4i w[QR];
#pragma unroll
      for (int u = 0; u < QR; u++) {
        const int lr = lr0 + 2 * (jb + u);
        w[u] = *(const lds_v4i*)(buf + lr * 512 + ((k ^ (lr & 31)) << 4));
      }
#pragma unroll
      for (int u = 0; u < QR; u++) {
        const int j = jb + u;
        const uint4 x = make_uint4((uint32_t)w[u].x, (uint32_t)w[u].y, (uint32_t)w[u].z,
                                   (uint32_t)w[u].w);
        const uint32_t sb = scale_byte_t<EL>(quad_max(chunk_absmax(x)));
        const uint2 pq = cvt8_t<EL>(x, sb);
        // block k / 4 of tile row tr0 + 64 h + 2 j
        if ((k & 3) == 0) sst[(tr0 + 64 * h + 2 * j) * 8 + (k >> 2)] = (uint8_t)sb;
        uint32_t off = 64 * h + 2 * j < lim ? off0 + (uint32_t)(64 * h + 2 * j) * rowq : OOB;
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_raw_buffer_store_b64((v2i){(int)pq.x, (int)pq.y}, rq, (int)off, 0, 0);
      }
    }
    __syncthreads();
  }
  // the tile's scales: row 64 wave + lane, 8 bytes at column block n0 / 32
  const int r = 64 * wave + lane;
  const v2i sv = *(const lds_v2i*)(sst + r * 8);
  uint32_t soff = r < (int)mrows ? (uint32_t)r * (uint32_t)lds_ + (uint32_t)(n0 >> 5) : OOB;
  asm volatile("" : "+v"(soff));
  __builtin_amdgcn_raw_buffer_store_b64(sv, rs, (int)soff, 0, 0);
}

// Linear workgroup id -> position t in the grouped tile order (GM_TILES
// m-tiles, n-tiles outer), so that the 32 tiles an XCD runs at once (8 along
// M x 4 along N) share A rows and B rows in that XCD's L2.  Workgroups are
// dealt to the 8 XCDs round-robin.  With few n-tiles (a group of GM_TILES
// m-tiles has at most 32 n-tiles, i.e. at most 8 runs of 32 tiles) run r of
// the order goes to XCD r % 8, so the XCDs work on one group at a time and
// read its A rows once from HBM between them; otherwise each XCD takes a
// contiguous eighth of the order (measured: 3-8% faster and 1.5% slower
// respectively than the other choice on the workload shapes), provided the
// eighths are whole multiples of GM_TILES tiles, so that an XCD's 32
// concurrent tiles line up with the groups; when they are not, the runs
// are dealt round-robin again (measured 1.6-3.2% faster at 7168 x 18432,
// whose eighths are 252 tiles).
__device__ __forceinline__ bool tile_runs_rr(uint32_t m, uint32_t n) {
  const uint32_t total = m * n;
  return n <= 32 || (total & 7) != 0 || ((total >> 3) % GM_TILES) != 0;
}

__device__ __forceinline__ void tile_of(int64_t bid, int64_t nm, int64_t nn, int64_t& mt,
                                        int64_t& nt) {
  // a grid has fewer than 2^24 workgroups of 256 threads (the host rejects
  // grids of 2^32 work-items), so tile indices fit in 32 bits
  const uint32_t b = (uint32_t)bid, m = (uint32_t)nm, n = (uint32_t)nn;
  const uint32_t total = m * n;
  const uint32_t x = b & 7, local = b >> 3;
  uint32_t t;
  if (tile_runs_rr(m, n)) {
    // runs of 32 round-robin over the XCDs; the tail past the last whole
    // 256 tiles keeps its position, so the map stays a bijection
    const uint32_t full = total & ~255u;
    t = b < full ? (((local >> 5) << 3) + x) * 32 + (local & 31) : b;
  } else {
    const uint32_t per = total >> 3, rem = total & 7;
    t = x * per + (x < rem ? x : rem) + local;
  }
  const uint32_t span = GM_TILES * n;
  const uint32_t group = t / span;
  const uint32_t first = group * GM_TILES;
  const uint32_t gsz = (m - first) < (uint32_t)GM_TILES ? (m - first) : (uint32_t)GM_TILES;
  const uint32_t in = t - group * span;
  const uint32_t q = in / gsz;
  mt = first + (in - q * gsz);
  nt = q;
}

}  // namespace mx
