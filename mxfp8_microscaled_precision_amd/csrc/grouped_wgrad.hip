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
// (16 cache lines instead of 64 for one step of 64 rows).  The kernel is
// persistent (one workgroup per compute unit walks its tiles): groups differ
// in length, so the experts are dealt longest first to groups of
// workgroups, each to the group with the least work so far; the workgroups
// on one XCD take contiguous runs of an expert's tile order so that tiles
// sharing rows share an L2.
#include "gemm_common.h"

namespace mx {

constexpr int W_STAGE = A_TILE + B_TILE;   // 64 KB of payload per K step
constexpr int W_SCALES = (BM + BN) * 16;   // A then B scales of four K steps: 8 KB
constexpr int W_MAX_GROUPS = 512;

// FA / FB: element formats of A (the gradient) and B (the input).
template <int FA, int FB>
struct WTile {
  u32x4 ra, rb;                     // the tile's whole rows of A and B
  u32x4 rsa, rsb;                   // their scale rows from the group's first column
  uint32_t kb;                      // the group's first column P
  uint32_t kb2;                     // the first column of the next tile's expert
  uint32_t voff_a, voff_b, rows32;  // chunk offset of this lane; offset of 32 rows
  uint32_t rows16;                  // scale offset of one row
  uint32_t svoff;                   // scale offset of this lane: row 64 wave + lane/4, step lane%4
  uint32_t pf_row, pf_a, pf_b;      // L2 prefetch: row offset, enable (0) or OOB
  int64_t nk;                       // K steps of the group
  bool odd;                         // nk odd: stage s lives in stage buffer (s + 1) % 2
  uint32_t nk2;                     // K steps of the next tile's expert (0: none)
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
  // and of B).  Past the group's end, the slots serve the workgroup's next
  // tile when it covers the same rows for a later expert (nk2 > 0): steps
  // kt = nk, nk + 1, nk + 2 fetch its first three steps, so its first
  // stages come from L2.  Either way two ops per call.
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

  // Stages 0 and 1 are requested together (a tile here runs only a few K
  // steps, so the second stage's latency would otherwise be paid once more
  // per tile): issue_first() loads stage 0 and the first scale group (24
  // ops per wave), issue_second() stage 1 and the next scale part (18 ops).
  __device__ __forceinline__ void issue_first(int wave, int lane) {
    issue(odd ? st1 : st0, 0, wave);
#pragma unroll
    for (int u = 0; u < 4; u++) issue_scales(0, u, wave, lane);
  }
  __device__ __forceinline__ void issue_second(int wave, int lane) {
    issue(odd ? st0 : st1, 1, wave);
    issue_scales(1, 0, wave, lane);  // the part step -1 would load
  }

  // The tile after issue_first() and issue_second(); `stored`: 32 stores
  // per wave were issued between the two.  Waits for stage 0 only (all but
  // the ops issued after it).  Steps past the group's end (nk == 0
  // included) touch no memory.
  __device__ __forceinline__ void run_issued(v16f (&acc)[4][4], int wave, int lane, bool stored) {
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
      for (int y = 0; y < 4; y++) acc[x][y] = (v16f){};
    if (stored)
      wait_vm<32 + 2 * CHUNKS + 2>();
    else
      wait_vm<2 * CHUNKS + 2>();
    __syncthreads();
    if (nk == 0) return;
    uint32_t sc_a[4], sc_b[4];
    v8i f0a[4], f0b[4], f1a[4], f1b[4];
    read_scales(0, wm, wn, lane, sc_a, sc_b);
    prefetch(2, wave);  // the steps' vmcnt(2) waits assume the latest two ops are prefetches
    read_frags<0>(odd ? st1 : st0, wm, wn, lane, f0a, f0b);
    // two copies of the step (a third for an odd tail would not fit the
    // registers): an odd step count enters the pair at its second step,
    // with the stages one buffer along (the prologue did what the skipped
    // step -1 would: stage 1's loads, the scale part, the prefetch)
    for (int64_t kt = odd ? -1 : 0; kt < nk; kt += 2) {
      if (kt >= 0) step(st0, st1, kt, wave, wm, wn, lane, sc_a, sc_b, f0a, f0b, f1a, f1b, acc);
      step(st1, st0, kt + 1, wave, wm, wn, lane, sc_a, sc_b, f0a, f0b, f1a, f1b, acc);
    }
  }
};

// Largest of the wave's values: the maximum within each row of 16 lanes by
// DPP (quad permutations, then rotations by 4 and 8 lanes), then over the
// four rows' lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_max(uint32_t m) {
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x124, 0xF, 0xF, false));  // row_ror:4
  m = umax(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x128, 0xF, 0xF, false));  // row_ror:8
  return umax(umax((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
              umax((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
}

// Work of one tile in K steps when experts are dealt to groups: its steps
// plus the fixed cost of starting and storing a tile.
constexpr uint32_t W_TILE_COST = 4;

// Persistent: the grid's workgroups walk the tiles (G experts x `per`
// output tiles of 256 x 256), so the expert order is worked out once per
// workgroup, no workgroup launch sits between two tiles, and the next tile
// of a workgroup is known while the current one runs (its first K steps are
// prefetched into L2 by the current tile's last steps).
//   groups > 0: the grid is groups x per workgroups; workgroup w keeps
//     output tile u = w % per of every expert dealt to its group w / per.
//     The experts, longest first (K steps descending, index ascending), go
//     one by one to the group with the least work so far (lowest index on
//     ties), which balances the groups the way list scheduling would.  Every
//     workgroup computes the same deal and keeps its own group's list.
//   groups == 0: workgroup w takes tiles w, w + grid, ... of the
//     expert-major tile order.
// Tile u of an expert: with per % 8 == 0 the workgroups on XCD x (w % 8)
// take the contiguous run x * per/8 .. of the expert's grouped tile order
// (GM_TILES m-tiles, n-tiles outer), so tiles that share rows share an L2.
template <int FA, int FB, bool OVERLAP>
__global__ void __launch_bounds__(NT)
grouped_wgrad_kernel(int64_t G, const int64_t* __restrict__ offsets, int64_t T, int64_t M,
                     int64_t N, int64_t ld, const uint8_t* __restrict__ a,
                     const uint8_t* __restrict__ sa, const uint8_t* __restrict__ b,
                     const uint8_t* __restrict__ sb, uint16_t* __restrict__ c, int groups) {
  __shared__ __attribute__((aligned(16))) uint8_t smem0[W_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t smem1[W_STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[2 * W_SCALES];
  __shared__ __attribute__((aligned(16))) uint8_t spf[2048];
  __shared__ int s_lo[W_MAX_GROUPS], s_hi[W_MAX_GROUPS];  // token ranges
  __shared__ uint32_t s_key[W_MAX_GROUPS];  // K steps << 9 | 511 - expert: distinct, larger first
  __shared__ short s_order[W_MAX_GROUPS];   // expert at each position of the longest-first order
  __shared__ short s_list[W_MAX_GROUPS];    // this workgroup's experts, in the order it runs them
  __shared__ int s_cnt;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nm = (M + BM - 1) / BM, nn = (N + BN - 1) / BN, per = nm * nn;
  const int64_t w = blockIdx.x, nwg = gridDim.x, tiles = G * per;
  // offsets clamped into [0, T]; a decrease reads as an empty group.  T is
  // below 2^23 (the token capacity limit), so ranges fit 32 bits and steps
  // 16 bits.
  for (int64_t g = threadIdx.x; g < G; g += NT) {
    int64_t lo = offsets[g], hi = offsets[g + 1];
    lo = lo < 0 ? 0 : (lo > T ? T : lo);
    hi = hi < lo ? lo : (hi > T ? T : hi);
    s_lo[g] = (int)lo;
    s_hi[g] = (int)hi;
    s_key[g] = ((uint32_t)((hi - lo + BK - 1) / BK) << 9) | (uint32_t)(511 - g);
  }
  __syncthreads();
  int cnt = 0;
  if (groups > 0) {
    for (int64_t g = threadIdx.x; g < G; g += NT) {
      const uint32_t k = s_key[g];
      int r = 0;
      for (int64_t h = 0; h < G; h++) r += s_key[h] > k ? 1 : 0;
      s_order[r] = (short)g;
    }
    __syncthreads();
    if (groups == 1) {
      // one group takes every expert, in the order
      for (int64_t p = threadIdx.x; p < G; p += NT) s_list[p] = s_order[p];
      cnt = (int)G;
      __syncthreads();
    } else {
      if (wave == 0) {
        // the order and each expert's work in registers (lane l of word m:
        // position 64 m + l), read back with readlane; lane j < groups
        // holds group j's work; the least loaded is the smallest
        // (work << 6 | j), found as the complement of a maximum
        int ord[W_MAX_GROUPS / 64];
        uint32_t wk[W_MAX_GROUPS / 64];
#pragma unroll
        for (int m = 0; m < W_MAX_GROUPS / 64; m++) {
          const int p = 64 * m + lane;
          ord[m] = p < G ? s_order[p] : 0;
          wk[m] = p < G ? (s_key[ord[m]] >> 9) + W_TILE_COST : 0u;
        }
        const int mine = (int)(w / per);
        uint32_t load = 0;
#pragma unroll
        for (int m = 0; m < W_MAX_GROUPS / 64; m++) {
          const int lim = (int)(G - 64 * m) < 64 ? (int)(G - 64 * m) : 64;
          for (int l = 0; l < lim; l++) {
            const int g = __builtin_amdgcn_readlane(ord[m], l);
            const uint32_t wg = (uint32_t)__builtin_amdgcn_readlane((int)wk[m], l);
            const uint32_t key = lane < groups ? (load << 6) | (uint32_t)lane : 0xFFFFFFFFu;
            const int j = (int)(~wave_max(~key) & 63u);
            if (lane == j) load += wg;
            if (j == mine) {
              if (lane == 0) s_list[cnt] = (short)g;
              cnt++;
            }
          }
        }
        if (lane == 0) s_cnt = cnt;
      }
      __syncthreads();
      cnt = s_cnt;
    }
  }
  const int64_t run = per >> 3;
  struct Cur {  // where a tile's result goes: expert, rows, first column
    int g;
    int64_t m0, m_end, n0;
  };
  struct Pos {  // output tile u of an expert: its tiles and prefetch duties
    uint32_t mt, nt;
    bool pfa, pfb;
  };
  // tile u's place in the grouped order; A is prefetched by a run's first
  // n-tile column, B by the first m-tile of each GM_TILES group (32-bit
  // arithmetic: per < 2^31)
  auto pos_of = [&](uint32_t u) -> Pos {
    const uint32_t un = (uint32_t)nn, um = (uint32_t)nm, ur = (uint32_t)run;
    const uint32_t L = (per & 7) == 0 ? (u & 7) * ur + (u >> 3) : u;
    const uint32_t first = L / (GM_TILES * un) * GM_TILES;
    const uint32_t gsz = (um - first) < GM_TILES ? (um - first) : GM_TILES;
    const uint32_t in = L % (GM_TILES * un);
    const uint32_t pos = (per & 7) == 0 ? (L % ur) : L;
    Pos p;
    p.mt = first + in % gsz;
    p.nt = in / gsz;
    p.pfa = pos < gsz;
    p.pfb = p.mt == first;
    return p;
  };
  // with groups, a workgroup keeps one output tile of every expert it runs
  const Pos fixed = pos_of((uint32_t)(w % per));
  // LDS values read at uniform addresses come back in vector registers;
  // readfirstlane keeps the tile's bookkeeping in scalar ones
  auto rfl = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  // tile k of this workgroup: its expert g and output tile, and the
  // workgroup's next tile's expert g2 when that covers the same rows (for
  // the L2 prefetch); sets up wt over them and cu; false past the last
  auto make = [&](int64_t k, WTile<FA, FB>& wt, Cur& cu) -> bool {
    int g, g2 = -1;
    int64_t u;
    if (groups > 0) {
      if (k >= cnt) return false;
      g = rfl(s_list[k]);
      u = w % per;
      if (k + 1 < cnt) g2 = rfl(s_list[k + 1]);
    } else {
      const int64_t t = w + k * nwg, tn = t + nwg;
      if (t >= tiles) return false;
      g = (int)(t / per);
      u = t - (int64_t)g * per;
      // the next tile reuses this one's rows when it is the same output tile
      if (tn < tiles && tn % per == u) g2 = (int)(tn / per);
    }
    const int64_t lo = rfl(s_lo[g]), hi = rfl(s_hi[g]);
    const int64_t lo2 = g2 >= 0 ? rfl(s_lo[g2]) : 0, hi2 = g2 >= 0 ? rfl(s_hi[g2]) : 0;
    const Pos ps = groups > 0 ? fixed : pos_of((uint32_t)u);
    const int64_t mt = ps.mt, nt = ps.nt;
    const int64_t P = 128 * (lo / 128 + g);
    const int64_t P2 = g2 >= 0 ? 128 * (lo2 / 128 + g2) : 0;
    wt.nk = (hi - lo + BK - 1) / BK;
    wt.odd = (wt.nk & 1) != 0;
    wt.nk2 = g2 >= 0 ? (uint32_t)((hi2 - lo2 + BK - 1) / BK) : 0u;
    wt.st0 = (lds_u8*)smem0;
    wt.st1 = (lds_u8*)smem1;
    wt.ss = (lds_u8*)sscale;
    wt.pf_scratch = (lds_u8*)spf;
    cu.g = g;
    cu.m0 = mt * BM;
    cu.n0 = nt * BN;
    cu.m_end = (cu.m0 + BM) < M ? cu.m0 + BM : M;
    const int64_t n_end = (cu.n0 + BN) < N ? cu.n0 + BN : N;
    wt.setup(a, sa, b, sb, ld, cu.m0, cu.m_end - cu.m0, cu.n0, n_end - cu.n0, P, P2, wave, lane);
    // prefetch only where a run first needs a slice
    wt.pf_a = ps.pfa ? 0u : OOB;
    wt.pf_b = ps.pfb ? 0u : OOB;
    return true;
  };
  // one WTile: after a tile's K loop it is set up over the next tile (the
  // store needs only the finished tile's place, kept in cc)
  WTile<FA, FB> wt;
  Cur cc;
  if (!make(0, wt, cc)) return;
  wt.issue_first(wave, lane);
  bool stored = false;
  for (int64_t k = 1;; k++) {
    wt.issue_second(wave, lane);
    v16f acc[4][4];
    wt.run_issued(acc, wave, lane, stored);
    // every load has landed (none may still be writing LDS) and every wave is
    // past its last read of the stage and scale buffers
    wait_vm_all();
    __syncthreads();
    Cur cn;
    const bool more = make(k, wt, cn);
    uint16_t* const ct = c + (int64_t)cc.g * M * N;
    if (OVERLAP) {
      // the next tile's stage 0 goes to stage buffer 0 while the result
      // leaves through buffer 1 (32 stores per wave); its stage 1 follows,
      // and it waits for stage 0 only: the stores drain under its first K
      // step
      if (more) wt.issue_first(wave, lane);
      // through the stage buffer the next tile's stage 0 does not use
      lds_u8* const sbuf = (more && wt.odd) ? (lds_u8*)smem0 : (lds_u8*)smem1;
      store_tile_bf16_lds_halves(acc, sbuf, ct, N, cc.m0, cc.m_end, cc.n0, N, wave & 1, wave >> 1,
                                 wave, lane);
      stored = true;
    } else {
      // (the store ends with a barrier: the next tile may reuse the stages)
      store_tile_bf16_lds(acc, (lds_u8*)smem0, (lds_u8*)smem1, ct, N, cc.m0, cc.m_end, cc.n0, N,
                          wave & 1, wave >> 1, wave, lane);
      if (more) wt.issue_first(wave, lane);
    }
    if (!more) break;
    cc = cn;
  }
}

hipError_t launch_grouped_wgrad(int a_elem, int b_elem, int64_t G, const int64_t* offsets, int64_t T,
                                int64_t M, int64_t N, int64_t cap, const void* a, const void* sa,
                                const void* b, const void* sb, void* c, int num_cus,
                                hipStream_t stream) {
  if (G < 1 || G > W_MAX_GROUPS || cap % BK != 0) return hipErrorInvalidValue;
  if ((a_elem != 0 && a_elem != 1) || (b_elem != 0 && b_elem != 1)) return hipErrorInvalidValue;
  const int64_t per = ((M + BM - 1) / BM) * ((N + BN - 1) / BN), tiles = G * per;
  if (tiles == 0) return hipSuccess;
  const int64_t cus = num_cus > 0 ? num_cus : 256;
  // groups of `per` workgroups when a whole number of them fits the chip
  // (and one wave can hold the groups' work); otherwise a plain walk
  int groups = 0;
  int64_t wgs;
  if (per <= cus && cus / per <= 64) {
    const int64_t m = (cus / per) < G ? cus / per : G;
    groups = (int)m;
    wgs = m * per;
  } else {
    wgs = cus < tiles ? cus : tiles;
    if (wgs >= 8) wgs = wgs / 8 * 8;  // keeps tile t on XCD t % 8
  }
  // the result leaves through one stage buffer while the other loads the
  // next tile (whole 8-column chunks, 32-bit store offsets)
  const bool overlap = N % 8 == 0 && (int64_t)BM * N * 2 < ((int64_t)1 << 31);
#define MX_WGRAD_LAUNCH(FA_, FB_, OV_)                                                            \
  hipLaunchKernelGGL((grouped_wgrad_kernel<FA_, FB_, OV_>), dim3((unsigned)wgs), dim3(NT), 0,     \
                     stream, G, offsets, T, M, N, cap, (const uint8_t*)a, (const uint8_t*)sa,    \
                     (const uint8_t*)b, (const uint8_t*)sb, (uint16_t*)c, groups)
#define MX_WGRAD_FMT(OV_)                                                                         \
  do {                                                                                            \
    if (a_elem == 0 && b_elem == 0) MX_WGRAD_LAUNCH(0, 0, OV_);                                   \
    else if (a_elem == 1 && b_elem == 0) MX_WGRAD_LAUNCH(1, 0, OV_);                              \
    else if (a_elem == 0 && b_elem == 1) MX_WGRAD_LAUNCH(0, 1, OV_);                              \
    else MX_WGRAD_LAUNCH(1, 1, OV_);                                                              \
  } while (0)
  if (overlap) MX_WGRAD_FMT(true);
  else MX_WGRAD_FMT(false);
#undef MX_WGRAD_FMT
#undef MX_WGRAD_LAUNCH
  return hipGetLastError();
}

}  // namespace mx
