// Per-expert weight gradient of the MoE backward for gfx950:
//   dW_g[m][n] = sum over the tokens t of expert group g of dY[t][m] * X[t][n]
// with both operands quantised in 32-token column blocks that restart at each
// group offset (MindSpeed RFC "add MXFP8-32x32 quantisation support to
// FSDP", section 2.2: grouped-matmul quantisation of the MoE experts'
// gate_up_proj / down_proj; the weight-gradient product is the backward half
// of that grouped matmul).  FP32 accumulation, BF16 result.
//
// Operands come from the grouped column quantisation: a [M, cap] and
// b [N, cap] with group g's tokens at columns P_g .. P_g + m_g - 1,
// P_g = 128 (o_g / 128 + g), and zero payload from there up to the next
// multiple of 128.  Every group's range therefore starts on a whole K step
// and the contraction over it runs whole 128-column steps with no masking;
// the scale row of a group starts on a 4-byte word.
//
// Tile 256 x 256 of one expert, four waves of 128 x 128, the MFMA layout and
// fragment reads of the dense GEMM; two LDS stages of payload.  Scales are
// staged per group of four K steps: a [256 rows][16 B] tile for A and one for
// B (four bytes per row per step), double-buffered, loaded with
// buffer_load_dword ... lds where one instruction covers 16 rows x 4 steps
// (16 cache lines instead of 64 for one step of 64 rows).  A workgroup runs
// one tile; groups differ in length, so
// the experts are taken longest first (up to 128 groups; the rank of each is
// counted in LDS) and the hardware's in-order dispatch balances the rest by
// giving the short tiles to the CUs that free up last; consecutive
// workgroups (dealt round-robin to the 8 XCDs) take contiguous runs of one
// expert's tile order per XCD so that tiles sharing rows share an L2.
#include "gemm_common.h"

namespace mx {

constexpr int W_STAGE = A_TILE + B_TILE;   // 64 KB of payload per K step
constexpr int W_SCALES = (BM + BN) * 16;   // A then B scales of four K steps: 8 KB
constexpr int W_MAX_GROUPS = 512;
constexpr int W_LPT_GROUPS = 128;           // longest-first expert order up to this many groups

// FA / FB: element formats of A (the gradient) and B (the input).
template <int FA, int FB>
struct WTile {
  u32x4 ra, rb, rsa, rsb;
  uint32_t voff_a, voff_b, rows32;  // chunk offset of this lane; offset of 32 rows
  uint32_t rows16;                  // scale offset of one row
  uint32_t svoff;                   // scale offset of this lane: row 64 wave + lane/4, step lane%4
  uint32_t pf_row, pf_a, pf_b;      // L2 prefetch: row offset, enable (0) or OOB
  int64_t nk;                       // K steps of the group
  lds_u8* st0;
  lds_u8* st1;
  lds_u8* ss;                       // two scale tiles of W_SCALES bytes
  lds_u8* pf_scratch;

  // Rows past the tile edge and columns past the group's range read zero.
  __device__ __forceinline__ void setup(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                        const uint8_t* sb, int64_t ld, int64_t m0, int64_t mrows,
                                        int64_t n0, int64_t nrows, int64_t P, int wave, int lane) {
    const int64_t lds = ld >> 5, span = BK * nk;
    ra = make_rsrc(a + m0 * ld + P, (mrows - 1) * ld + span);
    rb = make_rsrc(b + n0 * ld + P, (nrows - 1) * ld + span);
    rsa = make_rsrc(sa + m0 * lds + P / 32, (mrows - 1) * lds + 4 * nk);
    rsb = make_rsrc(sb + n0 * lds + P / 32, (nrows - 1) * lds + 4 * nk);
    // instruction t = wave + 4u covers LDS rows 8t .. 8t+7; lane i lands in
    // row 8t + i/8 at physical chunk i%8 holding logical chunk (i%8) ^ swz
    const int sw = (4 * wave + (lane >> 4)) & 7;
    voff_a = (uint32_t)((8 * wave + (lane >> 3)) * ld + 16 * ((lane & 7) ^ sw));
    voff_b = voff_a;
    rows32 = (uint32_t)(32 * ld);
    rows16 = (uint32_t)lds;
    svoff = (uint32_t)((64 * wave + (lane >> 2)) * lds + 4 * (lane & 3));
    pf_row = (uint32_t)((64 * wave + lane) * ld);
  }

  // Payload of K step kt into stage st; steps past the group's end get
  // out-of-range offsets and touch no memory.
  __device__ __forceinline__ void issue(lds_u8* st, int64_t kt, int wave) {
    const uint32_t base = kt < nk ? (uint32_t)(kt * BK) : OOB;
#pragma unroll
    for (int u = 0; u < CHUNKS; u++) dma16(st + (wave + 4 * u) * 1024, voff_a + base + u * rows32, ra);
#pragma unroll
    for (int u = 0; u < CHUNKS; u++)
      dma16(st + A_TILE + (wave + 4 * u) * 1024, voff_b + base + u * rows32, rb);
  }

  // Scales of step group q (steps 4q .. 4q+3), part u (0..3): rows
  // 64 wave + 16u .. +15 of A and of B, lane i -> row + i/4, step 4q + i%4,
  // into scale tile q % 2.  Steps at or past the group's end read zero (an
  // out-of-range offset): scale byte 0x00 is finite, and those steps' payload
  // is zero.
  __device__ __forceinline__ void issue_scales(int64_t q, int u, int wave, int lane) {
    const int64_t left = nk - 4 * q;  // steps of the group in range
    const int lim = left < 0 ? 0 : (left > 4 ? 4 : (int)left);
    const uint32_t base = (uint32_t)(16 * q) + (uint32_t)(16 * u) * rows16;
    const uint32_t off = (lane & 3) < lim ? svoff + base : OOB;
    lds_u8* tile = ss + (q & 1) * W_SCALES + (64 * wave + 16 * u) * 16;
    dma4(tile, off, rsa);
    dma4(tile + BM * 16, off, rsb);
  }

  __device__ __forceinline__ void prefetch(int64_t kt, int wave) {
    const uint32_t live = kt < nk ? 0u : OOB;
    const uint32_t kp = (uint32_t)(kt * BK);
    prefetch_lines(pf_scratch + wave * 512, (pf_row + kp) | pf_a | live, ra);
    prefetch_lines(pf_scratch + wave * 512 + 256, (pf_row + kp) | pf_b | live, rb);
  }

  // Scale words of step kt: bytes 2g, 2g+1 of the row's word for the step
  // are the step's blocks 2g and 2g+1, i.e. MFMA half S takes byte S.
  __device__ __forceinline__ void read_scales(int64_t kt, int wm, int wn, int lane, uint32_t* sar,
                                              uint32_t* sbr) {
    const int g = lane >> 5, i = lane & 31;
    const lds_u8* tile = ss + ((kt >> 2) & 1) * W_SCALES + 4 * (kt & 3) + 2 * g;
#pragma unroll
    for (int f = 0; f < 4; f++) sar[f] = *(const lds_u16*)(tile + (128 * wm + 32 * f + i) * 16);
#pragma unroll
    for (int f = 0; f < 4; f++) sbr[f] = *(const lds_u16*)(tile + BM * 16 + (128 * wn + 32 * f + i) * 16);
  }

  template <int S>
  __device__ __forceinline__ void read_frags(const lds_u8* st, int wm, int wn, int lane, v8i* af,
                                             v8i* bf) {
    const int g = lane >> 5, i = lane & 31;
#pragma unroll
    for (int f = 0; f < 4; f++) af[f] = read_frag(st, 128 * wm + 32 * f + i, S, g);
#pragma unroll
    for (int f = 0; f < 4; f++) bf[f] = read_frag(st + A_TILE, 128 * wn + 32 * f + i, S, g);
  }

  // One K step on stage `cur` (step kt), `nxt` holding step kt+1:
  //   phase A: MFMAs of K half 0, LDS reads of half 1 interleaved; then
  //     vmcnt(2) (all but this wave's two latest prefetches) and a barrier:
  //     step kt+1 has landed for every wave and nobody reads `cur` any more;
  //   phase B: scales and half-0 fragments of step kt+1, loads of step kt+2
  //     into `cur`, part (kt+1) % 4 of the scales of step group
  //     (kt+1) / 4 + 1, the prefetch of step kt+PF_DIST (always the last two
  //     vector-memory ops), MFMAs of half 1.
  // Group q's scales are loaded by steps 4q-5 .. 4q-2, so the last part has
  // landed at the barrier of step 4q-1, whose phase B first reads the group;
  // its tile was last read by step 4q-6, before the barrier of step 4q-5.
  __device__ __forceinline__ void step(lds_u8* cur, lds_u8* nxt, int64_t kt, int wave, int wm,
                                       int wn, int lane, uint32_t* sc_a, uint32_t* sc_b,
                                       v8i* f0a, v8i* f0b, v8i* f1a, v8i* f1b,
                                       v16f (&acc)[4][4]) {
    read_frags<1>(cur, wm, wn, lane, f1a, f1b);
    mma_tile<0, FA, FB>(f0a, f0b, sc_a, sc_b, acc);
    interleave_ops<16, 0>();
    wait_vm_but_prefetch();
    __syncthreads();
    uint32_t nx_a[4], nx_b[4];
    read_scales(kt + 1, wm, wn, lane, nx_a, nx_b);
    read_frags<0>(nxt, wm, wn, lane, f0a, f0b);
    issue(cur, kt + 2, wave);
    issue_scales((kt + 1) / 4 + 1, (int)((kt + 1) & 3), wave, lane);
    prefetch(kt + PF_DIST, wave);
    mma_tile<1, FA, FB>(f1a, f1b, sc_a, sc_b, acc);
    interleave_ops<24, 0>();
#pragma unroll
    for (int f = 0; f < 4; f++) {
      sc_a[f] = nx_a[f];
      sc_b[f] = nx_b[f];
    }
  }

  __device__ __forceinline__ void run(v16f (&acc)[4][4], int wave, int lane) {
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
      for (int y = 0; y < 4; y++) acc[x][y] = (v16f){};
    if (nk == 0) return;
    uint32_t sc_a[4], sc_b[4];
    v8i f0a[4], f0b[4], f1a[4], f1b[4];
    issue(st0, 0, wave);
#pragma unroll
    for (int u = 0; u < 4; u++) issue_scales(0, u, wave, lane);
    wait_vm_all();
    __syncthreads();
    read_scales(0, wm, wn, lane, sc_a, sc_b);
    issue(st1, 1, wave);
    issue_scales(1, 0, wave, lane);  // the part step -1 would load
    prefetch(2, wave);  // the steps' vmcnt(2) waits assume the latest two ops are prefetches
    read_frags<0>(st0, wm, wn, lane, f0a, f0b);
    // an even number of steps: a step past the end multiplies the zero
    // payload its out-of-range loads left in LDS (scale bytes 0x00, finite),
    // which is cheaper than a second copy of the step for the odd tail
    for (int64_t kt = 0; kt < nk; kt += 2) {
      step(st0, st1, kt, wave, wm, wn, lane, sc_a, sc_b, f0a, f0b, f1a, f1b, acc);
      step(st1, st0, kt + 1, wave, wm, wn, lane, sc_a, sc_b, f0a, f0b, f1a, f1b, acc);
    }
  }
};

template <int FA, int FB>
__global__ void __launch_bounds__(NT)
grouped_wgrad_kernel(int64_t G, const int64_t* __restrict__ offsets, int64_t T, int64_t M,
                     int64_t N, int64_t ld, const uint8_t* __restrict__ a,
                     const uint8_t* __restrict__ sa, const uint8_t* __restrict__ b,
                     const uint8_t* __restrict__ sb, uint16_t* __restrict__ c) {
  __shared__ __attribute__((aligned(16))) uint8_t smem0[W_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[W_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[2 * W_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t spf[2048];
  __shared__ int64_t s_nk[W_LPT_GROUPS];
  __shared__ int s_g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nm = (M + BM - 1) / BM, nn = (N + BN - 1) / BN, per = nm * nn;
  const int64_t t = blockIdx.x, pos_g = t / per, u = t % per;
  // Which expert: with at most W_LPT_GROUPS groups, position pos_g of the
  // experts ordered by K steps, longest first (ties by index), so the
  // longest tiles start first and the short ones fill in at the end;
  // otherwise expert pos_g.  Offsets are clamped as below.
  int64_t g = pos_g;
  if (G <= W_LPT_GROUPS) {
    for (int64_t gg = threadIdx.x; gg < G; gg += NT) {
      int64_t l = offsets[gg], r = offsets[gg + 1];
      l = l < 0 ? 0 : (l > T ? T : l);
      r = r < l ? l : (r > T ? T : r);
      s_nk[gg] = (r - l + BK - 1) / BK;
    }
    __syncthreads();
    for (int64_t gg = threadIdx.x; gg < G; gg += NT) {
      const int64_t k = s_nk[gg];
      int64_t rank = 0;
      for (int64_t j = 0; j < G; j++) {
        const int64_t kj = s_nk[j];
        rank += (kj > k || (kj == k && j < gg)) ? 1 : 0;
      }
      if (rank == pos_g) s_g = (int)gg;
    }
    __syncthreads();
    g = s_g;
  }
  // XCD x = u % 8 takes the contiguous run x * per/8 .. of the group's order
  const int64_t run = per >> 3;
  const int64_t L = (per & 7) == 0 ? (u & 7) * run + (u >> 3) : u;
  // grouped order inside the expert: GM_TILES m-tiles, n-tiles outer
  const int64_t first = L / (GM_TILES * nn) * GM_TILES;
  const int64_t gsz = (nm - first) < GM_TILES ? (nm - first) : GM_TILES;
  const int64_t in = L % (GM_TILES * nn);
  const int64_t mt = first + in % gsz, nt = in / gsz;
  // the group's token range (offsets clamped into [0, T]; a decrease reads as
  // an empty group)
  int64_t lo = offsets[g], hi = offsets[g + 1];
  lo = lo < 0 ? 0 : (lo > T ? T : lo);
  hi = hi < lo ? lo : (hi > T ? T : hi);
  const int64_t P = 128 * (lo / 128 + g);
  WTile<FA, FB> w;
  w.nk = (hi - lo + BK - 1) / BK;
  w.st0 = (lds_u8*)smem0;
  w.st1 = (lds_u8*)smem1;
  w.ss = (lds_u8*)sscale;
  w.pf_scratch = (lds_u8*)spf;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int64_t m_end = (m0 + BM) < M ? m0 + BM : M, n_end = (n0 + BN) < N ? n0 + BN : N;
  w.setup(a, sa, b, sb, ld, m0, m_end - m0, n0, n_end - n0, P, wave, lane);
  // prefetch only where a run first needs a slice: A by the run's first
  // n-tile column, B by the first m-tile of each GM_TILES group
  const int64_t pos = (per & 7) == 0 ? (L % run) : L;
  w.pf_a = pos < gsz ? 0u : OOB;
  w.pf_b = mt == first ? 0u : OOB;
  v16f acc[4][4];
  w.run(acc, wave, lane);
  wait_vm_all();  // no load may still be writing this workgroup's LDS when it ends
  store_tile_bf16(acc, c + g * M * N, N, m0, m_end, n0, N, wave & 1, wave >> 1, lane);
}

hipError_t launch_grouped_wgrad(int a_elem, int b_elem, int64_t G, const int64_t* offsets, int64_t T,
                                int64_t M, int64_t N, int64_t cap, const void* a, const void* sa,
                                const void* b, const void* sb, void* c, hipStream_t stream) {
  if (G < 1 || G > W_MAX_GROUPS || cap % BK != 0) return hipErrorInvalidValue;
  if ((a_elem != 0 && a_elem != 1) || (b_elem != 0 && b_elem != 1)) return hipErrorInvalidValue;
  const int64_t tiles = G * ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
#define MX_WGRAD_LAUNCH(FA_, FB_)                                                                 \
  hipLaunchKernelGGL((grouped_wgrad_kernel<FA_, FB_>), dim3((unsigned)tiles), dim3(NT), 0, stream, \
                     G, offsets, T, M, N, cap, (const uint8_t*)a, (const uint8_t*)sa,            \
                     (const uint8_t*)b, (const uint8_t*)sb, (uint16_t*)c)
  if (a_elem == 0 && b_elem == 0) MX_WGRAD_LAUNCH(0, 0);
  else if (a_elem == 1 && b_elem == 0) MX_WGRAD_LAUNCH(1, 0);
  else if (a_elem == 0 && b_elem == 1) MX_WGRAD_LAUNCH(0, 1);
  else MX_WGRAD_LAUNCH(1, 1);
#undef MX_WGRAD_LAUNCH
  return hipGetLastError();
}

}  // namespace mx
