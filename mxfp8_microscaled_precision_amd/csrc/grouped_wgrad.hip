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
  u32x4 ra, rb;                     // the tile's whole rows of A and B
  u32x4 rsa, rsb;                   // their scale rows from the group's first column
  uint32_t kb;                      // the group's first column P
  uint32_t kb2;                     // the first column of the expert prefetched for
  uint32_t voff_a, voff_b, rows32;  // chunk offset of this lane; offset of 32 rows
  uint32_t rows16;                  // scale offset of one row
  uint32_t svoff;                   // scale offset of this lane: row 64 wave + lane/4, step lane%4
  uint32_t pf_row, pf_a, pf_b;      // L2 prefetch: row offset, enable (0) or OOB
  int64_t nk;                       // K steps of the group
  uint32_t nk2;                     // K steps of the expert prefetched for (0: none)
  lds_u8* st0;
  lds_u8* st1;
  lds_u8* ss;                       // two scale tiles of W_SCALES bytes
  lds_u8* pf_scratch;

  // Rows past the tile edge and columns past the group's range read zero.
  __device__ __forceinline__ void setup(const uint8_t* a, const uint8_t* sa, const uint8_t* b,
                                        const uint8_t* sb, int64_t ld, int64_t m0, int64_t mrows,
                                        int64_t n0, int64_t nrows, int64_t P, int64_t P2, int wave,
                                        int lane) {
    // payload: whole rows (offsets past the tile's last row read zero;
    // columns past a group's tokens hold zero payload, the layout pads
    // every group's range to whole K steps, and steps past its end get
    // offset OOB), so one descriptor also serves the next expert's range
    const int64_t lds = ld >> 5;
    ra = make_rsrc(a + m0 * ld, mrows * ld);
    rb = make_rsrc(b + n0 * ld, nrows * ld);
    rsa = make_rsrc(sa + m0 * lds + P / 32, (mrows - 1) * lds + 4 * nk);
    rsb = make_rsrc(sb + n0 * lds + P / 32, (nrows - 1) * lds + 4 * nk);
    kb = (uint32_t)P;
    kb2 = (uint32_t)P2;
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
    const uint32_t base = kt < nk ? kb + (uint32_t)(kt * BK) : OOB;
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

  // L2 prefetch of K step kt (one line per row of this wave's 64 rows of A
  // and of B).  Past the group's end, the slots serve the expert whose tiles
  // the workgroups after this one on the XCD take over: steps kt = nk,
  // nk + 1, nk + 2 fetch its first three steps, so its first stages come
  // from L2.  Either way two ops per call.
  __device__ __forceinline__ void prefetch(int64_t kt, int wave) {
    const bool cur = kt < nk;
    const uint32_t j = (uint32_t)(kt - nk);  // step of the next expert
    const uint32_t live = (cur || (j < 3u && j < nk2)) ? 0u : OOB;
    // kb + kt BK on this group, kb2 + j BK on the next (modulo 2^32)
    const uint32_t off = pf_row + (cur ? kb : kb2 - (uint32_t)(nk * BK)) + (uint32_t)kt * BK;
    prefetch_lines(pf_scratch + wave * 512, off | pf_a | live, ra);
    prefetch_lines(pf_scratch + wave * 512 + 256, off | pf_b | live, rb);
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
    // half-0 fragments of step kt+1, each followed by two of the loads of
    // step kt+2 into `cur`, so the loads leave spread over the LDS reads
    // rather than as one burst that fills the address queue and holds up
    // the MFMAs behind it
    {
      const int g = lane >> 5, i = lane & 31;
      const uint32_t base = kt + 2 < nk ? kb + (uint32_t)((kt + 2) * BK) : OOB;
#pragma unroll
      for (int f = 0; f < 4; f++) {
        f0a[f] = read_frag(nxt, 128 * wm + 32 * f + i, 0, g);
        dma16(cur + (wave + 8 * f) * 1024, voff_a + base + 2 * f * rows32, ra);
        dma16(cur + (wave + 8 * f + 4) * 1024, voff_a + base + (2 * f + 1) * rows32, ra);
      }
#pragma unroll
      for (int f = 0; f < 4; f++) {
        f0b[f] = read_frag(nxt + A_TILE, 128 * wn + 32 * f + i, 0, g);
        dma16(cur + A_TILE + (wave + 8 * f) * 1024, voff_b + base + 2 * f * rows32, rb);
        dma16(cur + A_TILE + (wave + 8 * f + 4) * 1024, voff_b + base + (2 * f + 1) * rows32, rb);
      }
    }
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
    // Stages 0 and 1 are requested together (a tile here runs only a few
    // K steps, so the second stage's latency would otherwise be paid once
    // more per tile); the wait lets stage 1's 18 loads stay in flight.
    issue(st0, 0, wave);
#pragma unroll
    for (int u = 0; u < 4; u++) issue_scales(0, u, wave, lane);
    issue(st1, 1, wave);
    issue_scales(1, 0, wave, lane);  // the part step -1 would load
    wait_vm<2 * CHUNKS + 2>();  // all but stage 1's 16 payload and 2 scale loads
    __syncthreads();
    read_scales(0, wm, wn, lane, sc_a, sc_b);
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

// Largest of the wave's keys below `below` (0 if none): the maximum within
// each row of 16 lanes by DPP (quad permutations, then rotations by 4 and 8
// lanes), then over the four rows' lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_max_below(const uint32_t (&key)[2], uint32_t below) {
  uint32_t m = umax(key[0] < below ? key[0] : 0u, key[1] < below ? key[1] : 0u);
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
  return umax(umax((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
              umax((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
}

// The expert at position pos of the longest-first order (K steps
// descending, ties by index) and the one `ahead` positions further on, with
// their token ranges [lo, hi), found by each wave on its own without LDS or
// barriers: lane l holds experts l and 64 + l (G <= 128) as 24-bit keys
// (steps << 8 | 255 - index, all distinct, larger first).  A radix select
// walks the key bits, from the top bit of the largest key down, one ballot
// per bit, to the key with exactly `pos` larger keys; each later position is
// the largest key below the previous one.  Past the last expert, or with
// ahead == 0, g2 = -1.
// Offsets are clamped into [0, T] (a decrease reads as an empty group); T
// is below 2^23 (the token capacity limit), so steps fit 16 bits and ranges
// 32 bits.
__device__ __forceinline__ void lpt_experts(const int64_t* __restrict__ offsets, int64_t G, int64_t T,
                                            int64_t pos, int64_t ahead, int lane, int64_t& g,
                                            int64_t& lo, int64_t& hi, int64_t& g2, int64_t& lo2,
                                            int64_t& hi2) {
  int l[2], r[2];
  uint32_t key[2];
#pragma unroll
  for (int h = 0; h < 2; h++) {
    const int64_t gg = 64 * h + lane;
    int64_t a = 0, b = 0;
    if (gg < G) {
      a = offsets[gg];
      b = offsets[gg + 1];
    }
    a = a < 0 ? 0 : (a > T ? T : a);
    b = b < a ? a : (b > T ? T : b);
    l[h] = (int)a;
    r[h] = (int)b;
    // experts past G get key 0, below every real key (those are >= 128)
    key[h] = gg < G ? ((uint32_t)((b - a + BK - 1) / BK) << 8) | (uint32_t)(255 - gg) : 0u;
  }
  // the answer's bits above bit b are `prefix`; `want` keys larger than the
  // answer are still to be passed among the keys that share that prefix
  const uint32_t top = wave_max_below(key, 0xFFFFFFFFu);
  uint32_t prefix = 0;
  int want = (int)pos;
  for (int b = 31 - __builtin_clz(top | 1u); b >= 0; b--) {
    const uint32_t hi_half = (prefix >> b) | 1u;  // prefix with bit b set, shifted down
    const int cnt = __popcll(__ballot((key[0] >> b) == hi_half)) +
                    __popcll(__ballot((key[1] >> b) == hi_half));
    if (cnt > want)
      prefix |= 1u << b;
    else
      want -= cnt;
  }
  uint32_t next = ahead ? prefix : 0u;
  for (int64_t k = 0; k < ahead && next; k++) next = wave_max_below(key, next);
  const int idx = 255 - (int)(prefix & 255u), idx2 = 255 - (int)(next & 255u);
  g = idx;
  lo = __builtin_amdgcn_readlane(idx >> 6 ? l[1] : l[0], idx & 63);
  hi = __builtin_amdgcn_readlane(idx >> 6 ? r[1] : r[0], idx & 63);
  g2 = next ? idx2 : -1;
  lo2 = __builtin_amdgcn_readlane(idx2 >> 6 ? l[1] : l[0], idx2 & 63);
  hi2 = __builtin_amdgcn_readlane(idx2 >> 6 ? r[1] : r[0], idx2 & 63);
}

template <int FA, int FB>
__global__ void __launch_bounds__(NT)
grouped_wgrad_kernel(int64_t G, const int64_t* __restrict__ offsets, int64_t T, int64_t M,
                     int64_t N, int64_t ld, const uint8_t* __restrict__ a,
                     const uint8_t* __restrict__ sa, const uint8_t* __restrict__ b,
                     const uint8_t* __restrict__ sb, uint16_t* __restrict__ c, int xcd_cus) {
  __shared__ __attribute__((aligned(16))) uint8_t smem0[W_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[W_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[2 * W_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t spf[2048];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nm = (M + BM - 1) / BM, nn = (N + BN - 1) / BN, per = nm * nn;
  const int64_t t = blockIdx.x, pos_g = t / per, u = t % per;
  // Which expert: with at most W_LPT_GROUPS groups and fewer tiles per expert
  // than compute units, position pos_g of the experts ordered by K steps,
  // longest first (ties by index), so the longest tiles start first and the
  // short ones fill in at the end; otherwise expert pos_g.  lo, hi: its
  // token range.
  // XCD x = u % 8 takes the contiguous run x * per/8 .. of the group's order
  const int64_t run = per >> 3;
  // The workgroups that replace this one on its XCD's compute units take the
  // same run of the expert xcd_cus / run positions further on (an XCD runs
  // that many experts' runs at once); its first K steps are prefetched when
  // that is at most four positions on (0: no prefetch).
  int64_t ahead = (per & 7) == 0 ? (xcd_cus / run > 1 ? xcd_cus / run : 1) : 0;
  ahead = ahead <= 4 ? ahead : 0;
  int64_t g = pos_g, lo, hi, g2 = ahead ? pos_g + ahead : G, lo2 = 0, hi2 = 0;
  // When one expert's tiles occupy every compute unit at least once, each
  // expert is a round of its own and the order does not change the balance:
  // index order, no search.
  if (G <= W_LPT_GROUPS && per < 8 * (int64_t)xcd_cus) {
    lpt_experts(offsets, G, T, pos_g, ahead, lane, g, lo, hi, g2, lo2, hi2);
  } else {
    lo = offsets[g];
    hi = offsets[g + 1];
    lo = lo < 0 ? 0 : (lo > T ? T : lo);
    hi = hi < lo ? lo : (hi > T ? T : hi);
    if (g2 < G) {
      lo2 = offsets[g2];
      hi2 = offsets[g2 + 1];
      lo2 = lo2 < 0 ? 0 : (lo2 > T ? T : lo2);
      hi2 = hi2 < lo2 ? lo2 : (hi2 > T ? T : hi2);
    } else {
      g2 = -1;
    }
  }
  const int64_t L = (per & 7) == 0 ? (u & 7) * run + (u >> 3) : u;
  // grouped order inside the expert: GM_TILES m-tiles, n-tiles outer
  const int64_t first = L / (GM_TILES * nn) * GM_TILES;
  const int64_t gsz = (nm - first) < GM_TILES ? (nm - first) : GM_TILES;
  const int64_t in = L % (GM_TILES * nn);
  const int64_t mt = first + in % gsz, nt = in / gsz;
  const int64_t P = 128 * (lo / 128 + g);
  WTile<FA, FB> w;
  w.nk = (hi - lo + BK - 1) / BK;
  w.nk2 = g2 >= 0 ? (uint32_t)((hi2 - lo2 + BK - 1) / BK) : 0u;
  const int64_t P2 = g2 >= 0 ? 128 * (lo2 / 128 + g2) : 0;
  w.st0 = (lds_u8*)smem0;
  w.st1 = (lds_u8*)smem1;
  w.ss = (lds_u8*)sscale;
  w.pf_scratch = (lds_u8*)spf;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int64_t m_end = (m0 + BM) < M ? m0 + BM : M, n_end = (n0 + BN) < N ? n0 + BN : N;
  w.setup(a, sa, b, sb, ld, m0, m_end - m0, n0, n_end - n0, P, P2, wave, lane);
  // prefetch only where a run first needs a slice: A by the run's first
  // n-tile column, B by the first m-tile of each GM_TILES group
  const int64_t pos = (per & 7) == 0 ? (L % run) : L;
  w.pf_a = pos < gsz ? 0u : OOB;
  w.pf_b = mt == first ? 0u : OOB;
  v16f acc[4][4];
  w.run(acc, wave, lane);
  // every load has landed (none may still be writing LDS) and every wave is
  // past its last read of the stage buffers before they hold the result
  wait_vm_all();
  __syncthreads();
  store_tile_bf16_lds(acc, (lds_u8*)smem0, (lds_u8*)smem1, c + g * M * N, N, m0, m_end, n0, N,
                      wave & 1, wave >> 1, wave, lane);
}

hipError_t launch_grouped_wgrad(int a_elem, int b_elem, int64_t G, const int64_t* offsets, int64_t T,
                                int64_t M, int64_t N, int64_t cap, const void* a, const void* sa,
                                const void* b, const void* sb, void* c, int num_cus,
                                hipStream_t stream) {
  if (G < 1 || G > W_MAX_GROUPS || cap % BK != 0) return hipErrorInvalidValue;
  if ((a_elem != 0 && a_elem != 1) || (b_elem != 0 && b_elem != 1)) return hipErrorInvalidValue;
  const int64_t tiles = G * ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (tiles == 0) return hipSuccess;
  const int xcd_cus = (num_cus > 0 ? num_cus : 256) / 8;  // compute units per XCD
#define MX_WGRAD_LAUNCH(FA_, FB_)                                                                 \
  hipLaunchKernelGGL((grouped_wgrad_kernel<FA_, FB_>), dim3((unsigned)tiles), dim3(NT), 0, stream, \
                     G, offsets, T, M, N, cap, (const uint8_t*)a, (const uint8_t*)sa,            \
                     (const uint8_t*)b, (const uint8_t*)sb, (uint16_t*)c, xcd_cus)
  if (a_elem == 0 && b_elem == 0) MX_WGRAD_LAUNCH(0, 0);
  else if (a_elem == 1 && b_elem == 0) MX_WGRAD_LAUNCH(1, 0);
  else if (a_elem == 0 && b_elem == 1) MX_WGRAD_LAUNCH(0, 1);
  else MX_WGRAD_LAUNCH(1, 1);
#undef MX_WGRAD_LAUNCH
  return hipGetLastError();
}

}  // namespace mx
