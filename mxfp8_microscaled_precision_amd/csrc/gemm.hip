// MXFP8 GEMMs for gfx950: C[m][n] = sum_k A[m][k] * B[n][k] with E4M3
// operands, one E8M0 scale per 32 K-elements of each operand row, FP32
// accumulation and a BF16 result (torchtitan-npu MXFP8/HiF8 tutorial, "MXFP8
// / HiF8 architecture overview": the forward runs as an FP8 matmul whose
// output is restored to BF16; MoE experts run as a grouped matmul).  The
// grouped form multiplies rows offsets[g] .. offsets[g+1]-1 of the token
// matrix by expert g's weight (MindSpeed RFC "add MXFP8-32x32 quantisation
// support to FSDP", section 2.2: gate_up_proj / down_proj of MoE experts).
// The 32x32 weight variant takes one scale per 32x32 weight tile, and its
// backward-data product reads the one shared FP8 weight transposed (RFC
// sections 3.1 and 3.3.3).
//
// Hardware mapping (measured on the device):
//   v_mfma_scale_f32_32x32x64_f8f6f4, wave64.  Operand lane l holds row l%32;
//   lane half g = l/32 holds K bytes [16g, 16g+16) of scale block 0 and
//   [32+16g, 32+16g+16) of scale block 1; the scale of block b for row i is
//   the byte (op_sel) of lane i + 32b's scale register.  Result lane l, acc
//   j: row 8(j/4) + 4(l/32) + j%4, column l%32.
// The MFMA's first operand is B (our N side) and its second is A (our M
// side), so each lane ends with four consecutive n of one C row and stores 8
// bytes at a time.
//
// Workgroup tile 256 (M) x 256 (N), K step 128 bytes, four waves of 128x128
// (16 accumulators of 32x32 each).  Both operands are staged through a
// double-buffered LDS tile whose 16-byte chunks are XOR-swizzled by row, so
// the fragment reads (8 rows at one column per 128 bytes of LDS bandwidth)
// are conflict-free.
#include "mx_device.h"
#include "mx_kernels.h"

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int NT = 256;
constexpr int A_TILE = BM * BK;           // 32 KB
constexpr int B_TILE = BN * BK;           // 32 KB
constexpr int STAGE = A_TILE + B_TILE;    // 64 KB
constexpr int LDS_BYTES = 2 * STAGE;      // 128 KB
constexpr int CHUNKS = A_TILE / 16 / NT;  // 16-byte chunks per thread per operand: 8
constexpr int MAX_GROUPS = 512;

// Scale bytes of blocks kb0 .. kb0+3 of one operand row (blocks at or past
// nkb read as 0x7F = 2^0; their payload is zero).
__device__ __forceinline__ uint32_t load_scale4(const uint8_t* __restrict__ p, int64_t kb0,
                                                int64_t nkb) {
  if (kb0 + 4 <= nkb && (((uintptr_t)(p + kb0)) & 3) == 0) return *(const uint32_t*)(p + kb0);
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) r |= (uint32_t)(kb0 + i < nkb ? p[kb0 + i] : 0x7F) << (8 * i);
  return r;
}

// Tile scales of a transposed 32x32 weight: sb[kb][ncol32] for kb0 .. kb0+3.
__device__ __forceinline__ uint32_t load_scale4_t(const uint8_t* __restrict__ sb, int64_t kb0,
                                                  int64_t nkb, int64_t ld, int64_t ncol32) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; i++)
    r |= (uint32_t)(kb0 + i < nkb ? sb[(kb0 + i) * ld + ncol32] : 0x7F) << (8 * i);
  return r;
}

// Fragment of 32 rows x 64 K from a row-major LDS tile (128-byte rows).
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int s, int g) {
  const int x = row & 7;
  v4i lo = *(const v4i*)(tile + row * BK + (((2 * s + g) ^ x) << 4));
  v4i hi = *(const v4i*)(tile + row * BK + (((4 + 2 * s + g) ^ x) << 4));
  return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Fragment of 32 columns x 64 K from a [128 k][256 n] LDS tile (256-byte
// rows), read transposed with ds_read_b64_tr_b8: in each group of 16 lanes,
// lane 2r+h points at 8 bytes of row k+r and lane i receives byte i of the
// eight 16-byte rows, i.e. 8 consecutive k of column i.
__device__ __forceinline__ v8i read_frag_t(const uint8_t* tile, int nb, int s, int lane) {
  const int g = lane >> 5, q = (lane >> 4) & 1, r = (lane & 15) >> 1, hh = lane & 1;
  const int ncol = nb + 16 * q + 8 * hh;
  v2i p[4];
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const int k = (t >> 1) * 64 + 32 * s + 16 * g + (t & 1) * 8 + r;
    const uint8_t* a = tile + k * 256 + (((ncol >> 4) ^ (k & 7)) << 4) + (ncol & 15);
    p[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)a);
  }
  return (v8i){p[0].x, p[0].y, p[1].x, p[1].y, p[2].x, p[2].y, p[3].x, p[3].y};
}

template <int BMODE>
struct Tile {
  // operands
  const uint8_t* __restrict__ a;
  const uint8_t* __restrict__ sa;
  const uint8_t* __restrict__ b;
  const uint8_t* __restrict__ sb;
  uint16_t* __restrict__ c;
  int64_t m0, m_end, n0, N, K, nkb;
  uint8_t* smem;

  uint4 ra[CHUNKS], rb[CHUNKS];

  __device__ __forceinline__ void load_stage(int64_t k0) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < CHUNKS; u++) {
      const int id = u * NT + tid;
      const int row = id >> 3, cc = id & 7;
      int64_t m = m0 + row;
      m = m < m_end ? m : m_end - 1;
      const int64_t kb = k0 + 16 * cc;
      ra[u] = kb < K ? *(const uint4*)(a + m * K + kb) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < CHUNKS; u++) {
      const int id = u * NT + tid;
      if (BMODE == GEMM_B_TILE_T) {
        const int krow = id >> 4, cc = id & 15;
        const int64_t kk = k0 + krow, nn = n0 + 16 * cc;
        rb[u] = (kk < K && nn < N) ? *(const uint4*)(b + kk * N + nn) : make_uint4(0, 0, 0, 0);
      } else {
        const int row = id >> 3, cc = id & 7;
        int64_t n = n0 + row;
        n = n < N ? n : N - 1;
        const int64_t kb = k0 + 16 * cc;
        rb[u] = kb < K ? *(const uint4*)(b + n * K + kb) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store_stage(uint8_t* st) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < CHUNKS; u++) {
      const int id = u * NT + tid;
      const int row = id >> 3, cc = id & 7;
      *(uint4*)(st + row * BK + ((cc ^ (row & 7)) << 4)) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < CHUNKS; u++) {
      const int id = u * NT + tid;
      if (BMODE == GEMM_B_TILE_T) {
        const int krow = id >> 4, cc = id & 15;
        *(uint4*)(st + A_TILE + krow * 256 + ((cc ^ (krow & 7)) << 4)) = rb[u];
      } else {
        const int row = id >> 3, cc = id & 7;
        *(uint4*)(st + A_TILE + row * BK + ((cc ^ (row & 7)) << 4)) = rb[u];
      }
    }
  }

  // Scale registers for K step kb0: sar[fm] for the wave's A fragments and
  // sbr[fn] for its B fragments, already shifted so that byte s is the
  // scale of the block this lane half feeds in MFMA step s.
  __device__ __forceinline__ void load_scales(int64_t kb0, int wm, int wn, int lane,
                                              uint32_t* sar, uint32_t* sbr) {
    const int g = lane >> 5, i = lane & 31;
    const int64_t lda = K >> 5;
#pragma unroll
    for (int f = 0; f < 4; f++) {
      int64_t m = m0 + 128 * wm + 32 * f + i;
      m = m < m_end ? m : m_end - 1;
      sar[f] = load_scale4(sa + m * lda, kb0, nkb) >> (16 * g);
    }
#pragma unroll
    for (int f = 0; f < 4; f++) {
      int64_t n = n0 + 128 * wn + 32 * f + i;
      n = n < N ? n : N - 1;
      uint32_t v;
      if (BMODE == GEMM_B_ROW)
        v = load_scale4(sb + n * lda, kb0, nkb);
      else if (BMODE == GEMM_B_TILE)
        v = load_scale4(sb + (n >> 5) * lda, kb0, nkb);
      else
        v = load_scale4_t(sb, kb0, nkb, N >> 5, n >> 5);
      sbr[f] = v >> (16 * g);
    }
  }

  template <int S>
  __device__ __forceinline__ void mma_step(const uint8_t* st, int wm, int wn, int lane,
                                           const uint32_t* sar, const uint32_t* sbr,
                                           v16f (&acc)[4][4]) {
    const int g = lane >> 5, i = lane & 31;
    v8i af[4], bf[4];
#pragma unroll
    for (int f = 0; f < 4; f++) af[f] = read_frag(st, 128 * wm + 32 * f + i, S, g);
#pragma unroll
    for (int f = 0; f < 4; f++) {
      if (BMODE == GEMM_B_TILE_T)
        bf[f] = read_frag_t(st + A_TILE, 128 * wn + 32 * f, S, lane);
      else
        bf[f] = read_frag(st + A_TILE, 128 * wn + 32 * f + i, S, g);
    }
#pragma unroll
    for (int fn = 0; fn < 4; fn++)
#pragma unroll
      for (int fm = 0; fm < 4; fm++)
        acc[fn][fm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bf[fn], af[fm], acc[fn][fm], 0, 0, S, (int)sbr[fn], S, (int)sar[fm]);
  }

  __device__ __forceinline__ void run() {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    v16f acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
      for (int y = 0; y < 4; y++) acc[x][y] = (v16f){};
    const int64_t nk = (K + BK - 1) / BK;
    uint32_t sar[4], sbr[4], sar_n[4], sbr_n[4];
    load_stage(0);
    load_scales(0, wm, wn, lane, sar_n, sbr_n);
    store_stage(smem);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; kt++) {
#pragma unroll
      for (int f = 0; f < 4; f++) {
        sar[f] = sar_n[f];
        sbr[f] = sbr_n[f];
      }
      const bool more = kt + 1 < nk;
      if (more) {
        load_stage((kt + 1) * BK);
        load_scales((kt + 1) * (BK / 32), wm, wn, lane, sar_n, sbr_n);
      }
      const uint8_t* st = smem + (kt & 1) * STAGE;
      mma_step<0>(st, wm, wn, lane, sar, sbr, acc);
      mma_step<1>(st, wm, wn, lane, sar, sbr, acc);
      if (more) store_stage(smem + ((kt + 1) & 1) * STAGE);
      __syncthreads();
    }
    // epilogue: FP32 -> BF16 (RNE), four consecutive n per lane and row
    const int g = lane >> 5, i = lane & 31;
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int fn = 0; fn < 4; fn++) {
#pragma unroll
      for (int fm = 0; fm < 4; fm++) {
        const int64_t m = m0 + 128 * wm + 32 * fm + i;
        if (m >= m_end) continue;
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int64_t n = n0 + 128 * wn + 32 * fn + 8 * r4 + 4 * g;
          const v16f& v = acc[fn][fm];
          uint32_t h0 = bf16_rne(v[4 * r4 + 0]), h1 = bf16_rne(v[4 * r4 + 1]);
          uint32_t h2 = bf16_rne(v[4 * r4 + 2]), h3 = bf16_rne(v[4 * r4 + 3]);
          uint16_t* dst = c + m * N + n;
          if (vec_ok && n + 4 <= N) {
            *(uint2*)dst = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
          } else {
            if (n + 0 < N) dst[0] = (uint16_t)h0;
            if (n + 1 < N) dst[1] = (uint16_t)h1;
            if (n + 2 < N) dst[2] = (uint16_t)h2;
            if (n + 3 < N) dst[3] = (uint16_t)h3;
          }
        }
      }
    }
  }
};

// Linear workgroup id -> a contiguous run of tiles per XCD (workgroups are
// dealt to the 8 XCDs round-robin), then grouped M-major order inside the
// run so neighbouring tiles share A rows and B rows in that XCD's L2.
__device__ __forceinline__ void tile_of(int64_t bid, int64_t nm, int64_t nn, int64_t& mt,
                                        int64_t& nt) {
  const int64_t total = nm * nn;
  const int64_t x = bid & 7, local = bid >> 3;
  const int64_t per = total >> 3, rem = total & 7;
  const int64_t t = x * per + (x < rem ? x : rem) + local;
  constexpr int64_t GM = 8;
  const int64_t group = t / (GM * nn);
  const int64_t first = group * GM;
  const int64_t gsz = (nm - first) < GM ? (nm - first) : GM;
  const int64_t in = t % (GM * nn);
  mt = first + in % gsz;
  nt = in / gsz;
}

template <int BMODE>
__global__ void __launch_bounds__(NT)
gemm_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
            const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb, uint16_t* __restrict__ c,
            int64_t M, int64_t N, int64_t K) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  const int64_t nm = (M + BM - 1) / BM, nn = (N + BN - 1) / BN;
  int64_t mt, nt;
  tile_of(blockIdx.x, nm, nn, mt, nt);
  Tile<BMODE> t;
  t.a = a;
  t.sa = sa;
  t.b = b;
  t.sb = sb;
  t.c = c;
  t.m0 = mt * BM;
  t.m_end = (mt + 1) * BM < M ? (mt + 1) * BM : M;
  t.n0 = nt * BN;
  t.N = N;
  t.K = K;
  t.nkb = K >> 5;
  t.smem = smem;
  t.run();
}

// Persistent grouped GEMM: every workgroup derives the tile list from the
// device-side offsets (clamped into [0, T] and made non-decreasing, so bad
// offsets can never address outside the operands) and walks it with a static
// stride.  Tile t -> (group g, m tile within g, n tile).
__global__ void __launch_bounds__(NT)
grouped_gemm_kernel(int64_t G, const int64_t* __restrict__ offsets, int64_t T, int64_t N,
                    int64_t K, const uint8_t* __restrict__ a, const uint8_t* __restrict__ sa,
                    const uint8_t* __restrict__ b, const uint8_t* __restrict__ sb,
                    uint16_t* __restrict__ c) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  __shared__ int64_t s_off[MAX_GROUPS + 1];
  __shared__ int64_t s_pre[MAX_GROUPS + 1];
  const int64_t nn = (N + BN - 1) / BN;
  for (int64_t g = threadIdx.x; g <= G; g += NT) {
    int64_t o = offsets[g];
    s_off[g] = o < 0 ? 0 : (o > T ? T : o);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t prev = 0, acc = 0;
    for (int64_t g = 0; g < G; g++) {
      int64_t lo = s_off[g] > prev ? s_off[g] : prev;
      int64_t hi = s_off[g + 1] > lo ? s_off[g + 1] : lo;
      s_off[g] = lo;
      prev = lo;
      s_pre[g] = acc;
      acc += ((hi - lo + BM - 1) / BM) * nn;
    }
    s_off[G] = s_off[G] > prev ? s_off[G] : prev;
    s_pre[G] = acc;
  }
  __syncthreads();
  const int64_t total = s_pre[G];
  // contiguous tile runs per XCD
  const int64_t nwg = gridDim.x, bid = blockIdx.x;
  const int64_t wg = (bid & 7) * (nwg >> 3) + (bid >> 3);
  for (int64_t t = wg; t < total; t += nwg) {
    int64_t lo = 0, hi = G;  // largest g with s_pre[g] <= t
    while (hi - lo > 1) {
      int64_t mid = (lo + hi) >> 1;
      if (s_pre[mid] <= t) lo = mid; else hi = mid;
    }
    const int64_t g = lo;
    const int64_t local = t - s_pre[g];
    const int64_t mt = local / nn, nt = local % nn;
    Tile<GEMM_B_ROW> tl;
    tl.a = a;
    tl.sa = sa;
    tl.b = b + g * N * K;
    tl.sb = sb + g * N * (K >> 5);
    tl.c = c;
    tl.m0 = s_off[g] + mt * BM;
    tl.m_end = (tl.m0 + BM) < s_off[g + 1] ? tl.m0 + BM : s_off[g + 1];
    tl.n0 = nt * BN;
    tl.N = N;
    tl.K = K;
    tl.nkb = K >> 5;
    tl.smem = smem;
    tl.run();
  }
}

__global__ void fill_zero_kernel(uint4* __restrict__ p, int64_t n16, uint16_t* __restrict__ tail,
                                 int64_t ntail) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < ntail; i += blockDim.x) tail[i] = 0;
}

hipError_t launch_gemm(int bmode, int64_t M, int64_t N, int64_t K, const void* a, const void* sa,
                       const void* b, const void* sb, void* c, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid((unsigned)tiles), block(NT);
  const uint8_t *A = (const uint8_t*)a, *SA = (const uint8_t*)sa, *B = (const uint8_t*)b,
                *SB = (const uint8_t*)sb;
  uint16_t* C = (uint16_t*)c;
  switch (bmode) {
    case GEMM_B_ROW:
      hipLaunchKernelGGL(gemm_kernel<GEMM_B_ROW>, grid, block, 0, stream, A, SA, B, SB, C, M, N, K);
      break;
    case GEMM_B_TILE:
      hipLaunchKernelGGL(gemm_kernel<GEMM_B_TILE>, grid, block, 0, stream, A, SA, B, SB, C, M, N, K);
      break;
    case GEMM_B_TILE_T:
      hipLaunchKernelGGL(gemm_kernel<GEMM_B_TILE_T>, grid, block, 0, stream, A, SA, B, SB, C, M, N,
                         K);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(int64_t G, const int64_t* offsets, int64_t T, int64_t N, int64_t K,
                               const void* a, const void* sa, const void* b, const void* sb,
                               void* c, int num_cus, hipStream_t stream) {
  if (G > MAX_GROUPS) return hipErrorInvalidValue;
  const int64_t nn = (N + BN - 1) / BN;
  const int64_t upper = ((T + BM - 1) / BM + G) * nn;
  int64_t wgs = num_cus > 0 ? num_cus : 256;
  wgs = (wgs + 7) / 8 * 8;
  if (upper < wgs) wgs = (upper + 7) / 8 * 8;
  if (wgs < 8) wgs = 8;
  hipLaunchKernelGGL(grouped_gemm_kernel, dim3((unsigned)wgs), dim3(NT), 0, stream, G, offsets, T,
                     N, K, (const uint8_t*)a, (const uint8_t*)sa, (const uint8_t*)b,
                     (const uint8_t*)sb, (uint16_t*)c);
  return hipGetLastError();
}

hipError_t launch_fill_zero_bf16(void* c, int64_t n, hipStream_t stream) {
  int64_t n16 = n / 8, ntail = n - n16 * 8;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint4*)c, n16,
                     (uint16_t*)c + n16 * 8, ntail);
  return hipGetLastError();
}

}  // namespace mx
