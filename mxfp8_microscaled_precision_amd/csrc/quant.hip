// MX quantisation kernels for gfx950: BF16 -> E4M3 payload + E8M0 scales.
//
// Method: one E8M0 scale per 32 consecutive elements (1x32), computed from
// the block's absolute maximum on every call (dynamic), rceil rule, elements
// divided by the scale with round-to-nearest-even into E4M3 (torchtitan-npu
// MXFP8/HiF8 tutorial, "MXFP8 / HiF8 architecture overview", MXFP8 bullet;
// MindSpeed RFC "add MXFP8-32x32 quantisation support to FSDP", sections
// 3.3.1 and 3.3.3).  Dual-axis emits a forward copy blocked along the row and
// a backward copy blocked along the column from one read of x (tutorial,
// step-2 environment table, MXFP8_DUAL_AXIS_FORWARD; RFC section 3.3.3).  The
// 32x32 variant shares one scale per 32x32 tile (RFC sections 1.1, 3.1).
//
// The MoE backward needs column blocks along the token axis of every expert
// group: blocks restart at each group offset and the last block of a group
// holds only its remaining rows (MindSpeed RFC section 2.2: grouped-matmul
// quantisation of gate_up_proj / down_proj).  The grouped column mode writes
// group g's columns from P_g = 128 (o_g / 128 + g) on and fills every column
// that holds no token with zero blocks.
//
// All kernels are bound by HBM bandwidth: x is read once with 16-byte loads,
// every output byte is written once.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  u16x2 r = __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b));
  return __builtin_bit_cast(uint32_t, r);
}

// ---------------------------------------------------------------------------
// 1x32 along rows.  Row-major [R, C] with C % 32 == 0 is the same as the flat
// array cut into 32-element blocks, so the kernel walks 16-byte chunks of the
// flat array: four consecutive lanes hold one block.
// ---------------------------------------------------------------------------
constexpr int ROW_THREADS = 256;
constexpr int ROW_UNROLL = 4;

template <int EL>
__global__ void __launch_bounds__(ROW_THREADS)
quant_row_kernel(const uint4* __restrict__ x, uint2* __restrict__ q, uint8_t* __restrict__ s,
                 int64_t nchunks) {
  const int64_t span = (int64_t)ROW_THREADS * ROW_UNROLL;
  for (int64_t base = (int64_t)blockIdx.x * span; base < nchunks; base += (int64_t)gridDim.x * span) {
    uint4 v[ROW_UNROLL];
#pragma unroll
    for (int u = 0; u < ROW_UNROLL; u++) {
      int64_t c = base + u * ROW_THREADS + threadIdx.x;
      v[u] = c < nchunks ? load_stream16(x + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < ROW_UNROLL; u++) {
      int64_t c = base + u * ROW_THREADS + threadIdx.x;
      // quads are either wholly in range or wholly out (nchunks % 4 == 0)
      uint32_t sb = scale_byte_t<EL>(quad_max(chunk_absmax(v[u])));
      if (c < nchunks) {
        q[c] = cvt8_t<EL>(v[u], sb);
        if ((threadIdx.x & 3) == 0) s[c >> 2] = (uint8_t)sb;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 32x32 tiles.  A wave owns 32 rows x 128 columns (four tiles side by side):
// lane l = 16 r + c holds 16-byte chunk c of rows r, r + 4, ..., r + 28, so
// every load instruction reads 256 contiguous bytes of each of four rows and
// every store writes whole 128-byte lines of four payload rows.  A tile is
// the 16 lanes with the same c / 4; its amax is a quad reduction (DPP) and
// one exchange each with the lanes 16 and 32 away.  A workgroup of four
// waves covers 128 rows x 128 columns.
// ---------------------------------------------------------------------------
constexpr int B32_THREADS = 256;

template <int EL>
__global__ void __launch_bounds__(B32_THREADS)
quant_block32_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C, uint8_t* __restrict__ q,
                     uint8_t* __restrict__ s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, rg = lane >> 4;
  // 128 x 128 blocks, column blocks fastest (along the rows of x: measured
  // faster than down its columns)
  const int64_t lin = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
  const int64_t br = lin / gridDim.y, bc = lin - br * gridDim.y;
  const int64_t r0 = br * 128 + 32 * wave;
  const int64_t col = bc * 128 + 8 * c;
  // R and C are multiples of 32: a wave's 32 rows are all in or all out, and
  // so are a tile's four chunks
  if (r0 >= R) return;
  const bool live = col < C;
  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 8; i++)
    v[i] = live ? load_stream16(x + (r0 + rg + 4 * i) * C + col) : make_uint4(0, 0, 0, 0);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) m = umax(m, chunk_absmax(v[i]));
  m = quad_max(m);
  m = xor_max(m, 16);
  m = xor_max(m, 32);
  const uint32_t sb = scale_byte_t<EL>(m);
  if (!live) return;
#pragma unroll
  for (int i = 0; i < 8; i++) *(uint2*)(q + (r0 + rg + 4 * i) * C + col) = cvt8_t<EL>(v[i], sb);
  if (rg == 0 && (c & 3) == 0) s[(r0 >> 5) * (C >> 5) + (col >> 5)] = (uint8_t)sb;
}

// ---------------------------------------------------------------------------
// 2-D tile kernel for the column, dual-axis and grouped column modes.
//
// A workgroup of 8 waves covers 128 rows x 128 columns; wave w takes rows
// 32*(w/2) .. +32 and columns 64*(w%2) .. +64.  In a wave, lane l = 8g + h
// holds rows 4g .. 4g+3 and columns 8h .. 8h+7 as four 16-byte chunks, so
// - a row block (32 columns) spans the 4 lanes h = 4b .. 4b+3 of one quad,
// - a column block (32 rows) spans lanes h, h+8, ..., h+56 (xor 8, 16, 32).
// The column and dual modes stage their outputs in LDS (row payload
// [128 rows][128 B], column payload [128 columns][128 B], 16-byte chunks
// XOR-swizzled against bank conflicts, and both scale blocks) and then write
// every output row of the tile as whole 128-byte lines with 16-byte stores
// and the scales as dwords, instead of 8-, 4- and 1-byte pieces.
// ---------------------------------------------------------------------------
constexpr int TILE_THREADS = 512;
constexpr int TILE_ROWS = 128;
constexpr int TILE_COLS = 128;

enum TileMode { TILE_COL = 1, TILE_DUAL = 2, TILE_BLOCK32 = 3, TILE_GCOL = 4 };

typedef __attribute__((address_space(3))) uint8_t lds8;

// LDS tiles of 128 rows x 128 bytes; chunk k of row r lives at chunk k ^ sw(r).
__device__ __forceinline__ int row_chunk(int r, int k) { return k ^ ((r >> 2) & 7); }
__device__ __forceinline__ int col_chunk(int c, int k) { return k ^ ((c >> 3) & 7); }

// Grouped column mode: the wave's 32 output rows r0 .. r0+31 (a block of
// the padded token axis) -> first source row and number of real rows.  The
// group is the last g with P_g <= r0, found by counting (one ballot per 64
// groups, all offsets loaded at once, lane l of word k holding offsets[64k+l]);
// offsets are clamped into [0, T], so
// bad offsets give wrong blocks but only rows inside [0, T) are read.
constexpr int GCOL_MAX_GROUPS = 512;

// A wave-uniform lane's copy of a 64-bit register.
__device__ __forceinline__ int64_t readlane64(int64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void gcol_block(const int64_t* __restrict__ offsets, int64_t G,
                                           int64_t T, int64_t r0, int lane, int64_t& src,
                                           int& nreal) {
  int64_t o[GCOL_MAX_GROUPS / 64];
#pragma unroll
  for (int k = 0; k < GCOL_MAX_GROUPS / 64; k++) {
    const int64_t gg = 64 * k + lane;
    o[k] = gg <= G ? offsets[gg] : T;
  }
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < GCOL_MAX_GROUPS / 64; k++) {
    const int64_t gg = 64 * k + lane;
    const int64_t oc = o[k] < 0 ? 0 : (o[k] > T ? T : o[k]);
    cnt += __popcll(__ballot(gg < G && 128 * (oc / 128 + gg) <= r0));
  }
  src = 0;
  nreal = 0;
  if (cnt == 0) return;
  const int64_t g = cnt - 1;
  // offsets[g] and offsets[g + 1] from the lanes that loaded them (g is
  // uniform); only offsets[512] lies past the loaded words
  int64_t lo = 0, hi = 0;
#pragma unroll
  for (int k = 0; k < GCOL_MAX_GROUPS / 64; k++) {
    if ((g >> 6) == k) lo = readlane64(o[k], (int)(g & 63));
    if (((g + 1) >> 6) == k) hi = readlane64(o[k], (int)((g + 1) & 63));
  }
  if (g + 1 == GCOL_MAX_GROUPS) hi = offsets[g + 1];
  lo = lo < 0 ? 0 : (lo > T ? T : lo);
  hi = hi < lo ? lo : (hi > T ? T : hi);
  const int64_t first = 128 * (lo / 128 + g);
  if (r0 < first) return;                       // only with decreasing offsets
  const int64_t j = (r0 - first) >> 5;          // block of the group's range
  const int64_t left = (hi - lo) - 32 * j;
  src = lo + 32 * j;
  nreal = left <= 0 ? 0 : (left >= 32 ? 32 : (int)left);
}

// One 128 x 128 tile at rows R0.., columns C0.. (one tile per workgroup).
template <int MODE, int EL>
__device__ __forceinline__ void quant_tile(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                           uint8_t* __restrict__ q, uint8_t* __restrict__ s,
                                           uint8_t* __restrict__ qt, uint8_t* __restrict__ st,
                                           int64_t G, const int64_t* __restrict__ offsets,
                                           int64_t T, int64_t R0, lds8* LQ, lds8* LQT,
                                           lds8* LS, lds8* LST, int64_t C0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 3, h = lane & 7;
  const int wr = wave >> 1, wc = wave & 1;
  const int64_t r0 = R0 + 32 * wr;
  const int64_t c = C0 + 64 * wc + 8 * h;
  // R, C are multiples of 32: a wave's 32 rows are all in or all out, and
  // whole quads of columns are in or out
  const bool live = r0 < R && c < C;
  uint4 v[4];
  int nreal = 32;  // grouped column mode: rows 0 .. nreal-1 of the block are tokens
  if (MODE == TILE_GCOL) {
    int64_t src = 0;
    if (r0 < R) gcol_block(offsets, G, T, r0, lane, src, nreal);
#pragma unroll
    for (int i = 0; i < 4; i++)
      v[i] = (live && 4 * g + i < nreal) ? load_stream16(x + (src + 4 * g + i) * C + c)
                                         : make_uint4(0, 0, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++)
      v[i] = live ? load_stream16(x + (r0 + 4 * g + i) * C + c) : make_uint4(0, 0, 0, 0);
  }

  const int rl = 32 * wr + 4 * g;        // local row of this lane's first row
  const int cl = 64 * wc + 8 * h;        // local column of this lane's first column

  if (MODE == TILE_DUAL) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t sb = scale_byte_t<EL>(quad_max(chunk_absmax(v[i])));
      const int r = rl + i;
      const uint2 o = cvt8_t<EL>(v[i], sb);
      *(__attribute__((address_space(3))) u32x2*)(LQ + r * 128 + row_chunk(r, cl >> 4) * 16 +
                                                   (cl & 15)) = (u32x2){o.x, o.y};
      if ((h & 3) == 0) LS[r * 4 + (cl >> 5)] = (uint8_t)sb;
    }
  }

  // column maxima, two columns per packed word: cm[k] covers columns 2k, 2k+1
  const uint32_t M = 0x7FFF7FFFu;
  uint32_t cm[4];
  cm[0] = pk_max(pk_max(v[0].x & M, v[1].x & M), pk_max(v[2].x & M, v[3].x & M));
  cm[1] = pk_max(pk_max(v[0].y & M, v[1].y & M), pk_max(v[2].y & M, v[3].y & M));
  cm[2] = pk_max(pk_max(v[0].z & M, v[1].z & M), pk_max(v[2].z & M, v[3].z & M));
  cm[3] = pk_max(pk_max(v[0].w & M, v[1].w & M), pk_max(v[2].w & M, v[3].w & M));
#pragma unroll
  for (int k = 0; k < 4; k++) {
    cm[k] = pk_max(cm[k], (uint32_t)__shfl_xor((int)cm[k], 8, 64));
    cm[k] = pk_max(cm[k], (uint32_t)__shfl_xor((int)cm[k], 16, 64));
    cm[k] = pk_max(cm[k], (uint32_t)__shfl_xor((int)cm[k], 32, 64));
  }
  uint32_t sbc[8];
  // byte i of a column word is row 4g + i
  const uint32_t realmask = (4 * g + 0 < nreal ? 0x000000FFu : 0u) | (4 * g + 1 < nreal ? 0x0000FF00u : 0u) |
                            (4 * g + 2 < nreal ? 0x00FF0000u : 0u) | (4 * g + 3 < nreal ? 0xFF000000u : 0u);
#pragma unroll
  for (int k = 0; k < 4; k++) {
    sbc[2 * k] = scale_byte_t<EL>(cm[k] & 0xFFFFu);
    sbc[2 * k + 1] = scale_byte_t<EL>(cm[k] >> 16);
  }
  const uint32_t* w0 = (const uint32_t*)&v[0];
  const uint32_t* w1 = (const uint32_t*)&v[1];
  const uint32_t* w2 = (const uint32_t*)&v[2];
  const uint32_t* w3 = (const uint32_t*)&v[3];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int k = j >> 1;
    const uint32_t p01 = (j & 1) ? pair_hi(w0[k], w1[k]) : pair_lo(w0[k], w1[k]);
    const uint32_t p23 = (j & 1) ? pair_hi(w2[k], w3[k]) : pair_lo(w2[k], w3[k]);
    uint32_t out = sbc[j] == 0xFFu ? 0x7F7F7F7Fu : cvt4_t<EL>(p01, p23, cvt_scale(sbc[j]));
    if (MODE == TILE_GCOL) out &= realmask;  // rows that hold no token stay 0x00
    const int cc = cl + j;  // local column; 4 rows rl .. rl+3 of it
    *(__attribute__((address_space(3))) uint32_t*)(LQT + cc * 128 + col_chunk(cc, rl >> 4) * 16 +
                                                    (rl & 15)) = out;
  }
  // lane g keeps the scale of column cl + g
  uint32_t mine = sbc[0];
#pragma unroll
  for (int j = 1; j < 8; j++) mine = (g == j) ? sbc[j] : mine;
  LST[(cl + g) * 4 + wr] = (uint8_t)mine;
  __syncthreads();

  // write out: 16-byte chunks, 8 lanes per 128-byte output row
  const int t = threadIdx.x;
  const int64_t rows_here = (R - R0) < TILE_ROWS ? (R - R0) : TILE_ROWS;
  const int64_t cols_here = (C - C0) < TILE_COLS ? (C - C0) : TILE_COLS;
#pragma unroll
  for (int u = 0; u < 2; u++) {
    const int id = t + TILE_THREADS * u;
    const int row = id >> 3, k = id & 7;
    if (row < cols_here && 16 * k < rows_here) {  // column payload -> q_t rows
      const u32x4 d = *(const __attribute__((address_space(3))) u32x4*)(
          LQT + row * 128 + col_chunk(row, k) * 16);
      __builtin_nontemporal_store(d, (u32x4*)(qt + (C0 + row) * R + R0 + 16 * k));
    }
    if (MODE == TILE_DUAL && row < rows_here && 16 * k < cols_here) {  // row payload -> q rows
      const u32x4 d = *(const __attribute__((address_space(3))) u32x4*)(
          LQ + row * 128 + row_chunk(row, k) * 16);
      __builtin_nontemporal_store(d, (u32x4*)(q + (R0 + row) * C + C0 + 16 * k));
    }
  }
  // scales: four consecutive blocks per row / column
  if (t < TILE_COLS && t < cols_here) {
    uint8_t* dst = st + (C0 + t) * (R >> 5) + (R0 >> 5);
    const int nb = (int)(rows_here >> 5);
    if (nb == 4 && ((uintptr_t)dst & 3) == 0) {
      *(uint32_t*)dst = *(const __attribute__((address_space(3))) uint32_t*)(LST + t * 4);
    } else {
      for (int b = 0; b < nb; b++) dst[b] = LST[t * 4 + b];
    }
  }
  if (MODE == TILE_DUAL && t >= 256 && t - 256 < rows_here) {
    const int r = t - 256;
    uint8_t* dst = s + (R0 + r) * (C >> 5) + (C0 >> 5);
    const int nb = (int)(cols_here >> 5);
    if (nb == 4 && ((uintptr_t)dst & 3) == 0) {
      *(uint32_t*)dst = *(const __attribute__((address_space(3))) uint32_t*)(LS + r * 4);
    } else {
      for (int b = 0; b < nb; b++) dst[b] = LS[r * 4 + b];
    }
  }
}

// grid.z indexes a batch of equally shaped matrices (contiguous inputs and
// outputs); the grouped column mode uses G, offsets and T (x has T rows, R is
// the padded capacity).  One tile per workgroup in every mode.
template <int MODE, int EL>
__global__ void __launch_bounds__(TILE_THREADS)
quant_tile_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C, uint8_t* __restrict__ q,
                  uint8_t* __restrict__ s, uint8_t* __restrict__ qt, uint8_t* __restrict__ st,
                  int64_t G, const int64_t* __restrict__ offsets, int64_t T) {
  if (blockIdx.z) {
    const int64_t z = blockIdx.z, n = R * C;
    x += z * n;
    q += q ? z * n : 0;
    s += s ? z * (n >> 5) : 0;
    qt += qt ? z * n : 0;
    st += st ? z * (n >> 5) : 0;
  }
  __shared__ __attribute__((aligned(16))) uint8_t lq[TILE_ROWS * 128];   // row payload
  __shared__ __attribute__((aligned(16))) uint8_t lqt[TILE_COLS * 128];  // column payload
  __shared__ __attribute__((aligned(16))) uint8_t ls[TILE_ROWS * 4];     // row scales
  __shared__ __attribute__((aligned(16))) uint8_t lst[TILE_COLS * 4];    // column scales
  // dispatch order (measured): the column modes go along the rows of x,
  // column tiles fastest, so that the 32 row tiles sharing each line of the
  // column-scale array run close together and the line leaves L2 whole; the
  // dual mode down its columns, row tiles fastest (as the grid is laid out)
  int64_t tr = blockIdx.x, tc = blockIdx.y;
  if (MODE == TILE_COL || MODE == TILE_GCOL) {
    const int64_t lin = (int64_t)blockIdx.x + (int64_t)blockIdx.y * gridDim.x;
    tr = lin / gridDim.y;
    tc = lin - tr * gridDim.y;
  }
  quant_tile<MODE, EL>(x, R, C, q, s, qt, st, G, offsets, T, tr * TILE_ROWS, (lds8*)lq, (lds8*)lqt,
                       (lds8*)ls, (lds8*)lst, tc * TILE_COLS);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_quant_row(const void* x, int64_t n, void* q, void* s, int elem,
                            hipStream_t stream) {
  int64_t nchunks = n / 8;
  int64_t span = (int64_t)ROW_THREADS * ROW_UNROLL;
  int64_t blocks = (nchunks + span - 1) / span;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  if (elem == ELEM_E5M2)
    hipLaunchKernelGGL(quant_row_kernel<ELEM_E5M2>, dim3((unsigned)blocks), dim3(ROW_THREADS), 0,
                       stream, (const uint4*)x, (uint2*)q, (uint8_t*)s, nchunks);
  else
    hipLaunchKernelGGL(quant_row_kernel<ELEM_E4M3>, dim3((unsigned)blocks), dim3(ROW_THREADS), 0,
                       stream, (const uint4*)x, (uint2*)q, (uint8_t*)s, nchunks);
  return hipGetLastError();
}

template <int MODE, int EL>
static void launch_tile(dim3 grid, const void* x, int64_t R, int64_t C, void* q, void* s, void* qt,
                        void* st, int64_t G, const int64_t* offsets, int64_t T, hipStream_t stream) {
  hipLaunchKernelGGL((quant_tile_kernel<MODE, EL>), grid, dim3(TILE_THREADS), 0, stream,
                     (const uint16_t*)x, R, C, (uint8_t*)q, (uint8_t*)s, (uint8_t*)qt, (uint8_t*)st,
                     G, offsets, T);
}

template <int MODE>
static void launch_tile_elem(int elem, dim3 grid, const void* x, int64_t R, int64_t C, void* q,
                             void* s, void* qt, void* st, int64_t G, const int64_t* offsets,
                             int64_t T, hipStream_t stream) {
  if (elem == ELEM_E5M2)
    launch_tile<MODE, ELEM_E5M2>(grid, x, R, C, q, s, qt, st, G, offsets, T, stream);
  else
    launch_tile<MODE, ELEM_E4M3>(grid, x, R, C, q, s, qt, st, G, offsets, T, stream);
}

hipError_t launch_quant_tile(int mode, const void* x, int64_t R, int64_t C, void* q, void* s,
                             void* qt, void* st, int64_t batch, int elem, hipStream_t stream) {
  dim3 grid((unsigned)((R + TILE_ROWS - 1) / TILE_ROWS), (unsigned)((C + TILE_COLS - 1) / TILE_COLS),
            (unsigned)batch);
  switch (mode) {
    case TILE_COL:
      launch_tile_elem<TILE_COL>(elem, grid, x, R, C, q, s, qt, st, 0, nullptr, 0, stream);
      break;
    case TILE_DUAL:
      launch_tile_elem<TILE_DUAL>(elem, grid, x, R, C, q, s, qt, st, 0, nullptr, 0, stream);
      break;
    case TILE_BLOCK32: {
      // one 256-thread workgroup per 128 x 128 block (grid.z == 1: a batch of
      // 32x32-tiled matrices is one stacked matrix)
      if (batch != 1) return hipErrorInvalidValue;
      if (elem == ELEM_E5M2)
        hipLaunchKernelGGL(quant_block32_kernel<ELEM_E5M2>, dim3(grid.x, grid.y), dim3(B32_THREADS), 0,
                           stream, (const uint16_t*)x, R, C, (uint8_t*)q, (uint8_t*)s);
      else
        hipLaunchKernelGGL(quant_block32_kernel<ELEM_E4M3>, dim3(grid.x, grid.y), dim3(B32_THREADS), 0,
                           stream, (const uint16_t*)x, R, C, (uint8_t*)q, (uint8_t*)s);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_grouped_col(const void* x, int64_t T, int64_t C, int64_t G,
                                    const int64_t* offsets, int64_t cap, void* qt, void* st,
                                    int elem, hipStream_t stream) {
  if (G < 1 || G > GCOL_MAX_GROUPS) return hipErrorInvalidValue;
  dim3 grid((unsigned)((cap + TILE_ROWS - 1) / TILE_ROWS), (unsigned)((C + TILE_COLS - 1) / TILE_COLS));
  launch_tile_elem<TILE_GCOL>(elem, grid, x, cap, C, nullptr, nullptr, qt, st, G, offsets, T, stream);
  return hipGetLastError();
}

}  // namespace mx
