// Expert projections for many rows per expert (prefill), with fragment-order
// or row-major weights: both grouped GEMMs of the Mixtral sparse-MoE block
// (nnterp Mixtral page, support(): the down projection receives act(gate) *
// up with act = SiLU; the experts are one stacked module), the first fused
// with that activation, as in ffn_bf16.hip:
//
//   gate/up: h[p, n] = silu(sum_i x[r,i] w1[e,n,i]) * (sum_i x[r,i] w3[e,n,i]),
//            r = sorted_asg[p] / k for p in expert e's grouped rows; h is bf16;
//   down:    y[p, n] = sum_i h[p,i] w2[e,n,i], float32, optionally split in K
//            into two partial sums over [0, ksplit) and [ksplit, K) (written
//            to part[0] and part[1]; y is their sum in that order), the split
//            chosen on the device from the expert counts (below).
//
// Tile: 256 weight rows x 256 token rows per workgroup of 8 waves, two per
// SIMD (so one wave's MFMAs run while the other waits on a load issue or the
// barrier); wave (wn, wm), wn = 0..3, wm = 0..1, owns 64 weight rows and
// tokens 128 wm .. 128 wm + 127: a 4 x 8 grid of 16x16 MFMA tiles (128
// accumulator registers). For gate/up the 64 rows are 32 w1 rows and the same
// 32 w3 rows (w1 and w3 rows n .. n+127 per tile, n = 128 nt), so gate and up
// of one h column meet in one lane; for down they are w2 rows 256 nt + 64 wn
// .. + 63. K advances in 32-wide steps.
//
// Both operands go global -> LDS with the 16-byte direct-to-LDS buffer loads,
// no register staging. Fragment-order weights (template parameter PACKED;
// row-major weights below): one load instruction moves one 1 KiB MFMA
// fragment (one contiguous KiB of the fragment-order matrix) into LDS in lane
// order; four 16 KiB buffers hold the weight fragments of steps t .. t+3.
// Tokens: one load instruction moves 8 token rows x 128 bytes (gathered rows
// of x for gate/up, grouped rows of h for down), whole cache lines covering
// two K steps (half the L2 requests of 16 rows x 64 bytes, which measured
// 13-15% slower); two 32 KiB buffers hold 64-wide K stages of the 256 rows,
// row-major, with the 16-byte chunk c of row r stored in slot c ^ ((r / 2) %
// 8), so that every MFMA fragment read (16 rows, one chunk) touches 16
// distinct bank groups. Weight loads of step t+4 go out in step t (three
// steps of lead), token loads of stage (t+3)/2 in odd steps t (two steps of
// lead), tokens before weights so that the in-order load counter never makes
// a wait cover a younger weight load. The only waits are one "vmcnt <= 4"
// (odd steps) or "<= 8" (even steps) and one barrier per step.
//
// Per step a wave runs 8 groups of 4 MFMAs; groups 0-3 also read three
// fragments each of step t+1 into the second register set (in the order the
// next step uses them) and issue the step's loads. Groups are closed by
// scheduling barriers and this file is built with the machine scheduler off:
// that keeps the interleaving as written, and it lets the register allocator
// keep every accumulator in one place (the scheduler's reordering otherwise
// makes it rotate the accumulators through copies).
//
// Token tiles that run past an expert's rows: each wave computes only its
// token fragments that hold a row (rounded up to an even count; a template
// parameter, so the loop stays branch-free), and still issues all loads and
// barriers with the other waves.
//
// Row-major weights (template parameter PACKED false): the weight rows are
// staged as the token rows are (8 rows x 128 bytes per load, swizzled 32 KiB
// K64 stages) and the weight fragments are read like the token fragments.
// Three weight stages (160 KiB of LDS in all): the loads of weight stage
// (t+5)/2 go out in odd steps t after the token loads of stage (t+3)/2, four
// steps of lead (with two stages, two steps of lead and a full drain per
// stage measured 1-4% slower); the only waits are "vmcnt <= 4" in odd steps
// and none in even ones, plus the barrier. The loop is unrolled over the 12
// steps of a buffer cycle so that every buffer index is a constant; the 4 or
// 8 steps left after the last whole cycle run with the first cycle's
// indices. The MFMAs, their operands and their order are those of the
// fragment-order kernel, so the results of the two layouts are identical.
//
// Row scales (template parameter SCALED, fragment order only: weight-only
// int8 codes the caller has widened to exact bfloat16): the finished float32
// sums are multiplied by their weight row's scale from arrays [E, N] before
// the SiLU*mul (gate by the w1 row's scale, up by the w3 row's) or the store
// (down, each K-split partial), as the int8 decode kernels do.
//
// Paired last m-tiles (fragment-order weights): an expert's last m-tile of at
// most 128 rows costs nearly as much as a full one (its time is set by the
// weight stream it shares with the full tiles of its weight tile, not by its
// own loads or MFMAs: halving either changed nothing, while leaving those
// tiles out took 9-13% off the launch), so two weight tiles of an XCD share
// one: 512 weight rows x 128 token rows, each wave the same 64 x 128 block as
// in a 256x256 tile. Gate/up always pairs them (8x7B prefill: 4032 -> 3808
// tiles, 1574 -> 1497-1544 us; 8x22B 1510 -> 1458 us). The down projection
// pairs them while experts average at most two m-tiles (T*k <= 512 E), where
// last m-tiles are a large share of its few tiles (32 experts at 4096 tokens:
// 1099 vs 1139 us unsplit, 1035 us with the split below; 16 experts: 856-889
// vs about 910 us); with more rows per expert pairing measured 0-2% slower.
//
// Every output element is one float32 MFMA accumulation over its K range in
// increasing K, 32 at a time: the order of the 128-row tiled kernels, whose
// results this kernel reproduces bit for bit.
//
// All loads go through buffer descriptors bounded to the source array, so an
// offset outside it reads zeros instead of faulting (the host checks that the
// byte offsets fit in 31 bits; inside the kernel they are in range by
// construction: token rows are clamped to the expert's last row).
#include "common.h"

namespace moe {
namespace {

typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int DT = 256;             // weight rows and token rows per tile
constexpr int kFragE = 512;         // bf16 elements per 16x32 fragment (1 KiB)
constexpr int kWBufE = 16 * kFragE; // one K32 step of the 16 weight fragments (16 KiB)
constexpr int kTBufE = DT * 64;     // one K64 stage of the 256 token rows (32 KiB)
constexpr int kDmaThreads = 512;
// buffer descriptor word 3 (gfx9): 32-bit data format, for raw dword loads
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt not waited on
constexpr int vmcnt_le(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// workgroup -> (expert e, its first grouped row beg and row count M, token
// tile m0, weight tile nt, K part sp); workgroup b runs on XCD x = b % 8.
// When the weight tiles come in multiples of 8 (every real shape), XCD x
// takes the weight tiles nt = x, x + 8, ... of every expert and K part, each
// with all its m-tiles: every XCD then gets the same share of every expert's
// rows, part-filled last m-tiles included (contiguous slices of an
// expert-major list gave XCDs with several nearly empty last tiles 12% less
// work than others), and the m-tiles sharing a weight tile run together in
// one XCD's L2. Its tiles are listed K part by K part (the longer first part
// of every tile before any second part, so that the short ones fill the last
// round), expert by expert, and taken in that order, tile q by workgroup
// 8q + x. Within an expert, the XCD's weight
// tiles go in pairs (2g, 2g+1) whose m-tiles alternate (the weight tiles of
// a pair are then read by tiles running together: L2 hits 0.55 -> 0.75 for
// gate/up with the paired tiles below; 8x22B down 766 -> 741 us); with
// pair_tails, an expert whose last m-tile holds at most DT/2 rows puts one
// tile for both weight tiles' last m-tiles first in each pair's group (nt2 =
// the second weight tile; otherwise nt2 = -1); an odd weight tile left over
// comes last with its m-tiles in order. Otherwise (fewer or
// ragged weight tiles) XCD x takes the x-th of 8 equal slices of the list of
// all tiles, expert by expert, K part, n-tile, m-tile. Surplus workgroups of
// the worst-case grid return.
//
// Finding the workgroup's expert: every wave of the workgroup does it on its
// own, one expert per lane (E <= 32), so no wave walks the experts in scalar
// code (eight waves doing that share the CU's scalar unit: at 32 experts the
// walk, and the split choice below, cost several microseconds per tile).

// one XCD's tile list of one K part, lane l < E holding expert l: its grouped
// rows ml and first row bl, its tiles cl and their inclusive prefix sum il
// over the lanes; n = all the tiles
struct XcdList {
  int ml, bl, cl, il, n;
};

// tiles of one expert of ml rows in an XCD's list (nnx weight tiles per XCD)
__device__ __forceinline__ int expert_tiles(int ml, int nnx, bool pair_tails) {
  const int pairs = nnx >> 1;
  const int mt = (ml + DT - 1) / DT;
  const bool small = pair_tails && pairs > 0 && mt > 0 && ml - (mt - 1) * DT <= DT / 2;
  return small ? pairs * (2 * mt - 1) + (nnx - 2 * pairs) * mt : nnx * mt;
}

// inclusive prefix sum over lanes 0..31 (lane 31: the total of lanes 0..31)
__device__ __forceinline__ int prefix32(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ __forceinline__ XcdList xcd_list(const int32_t* __restrict__ offsets, int E, int ntn,
                                            bool pair_tails) {
  const int lane = threadIdx.x & (kWave - 1);
  XcdList L;
  const bool in = lane < E;
  L.bl = in ? offsets[lane] : 0;
  L.ml = in ? offsets[lane + 1] - L.bl : 0;
  L.cl = expert_tiles(L.ml, ntn >> 3, pair_tails);
  L.il = prefix32(L.cl, lane);
  L.n = __builtin_amdgcn_readfirstlane(__shfl(L.il, 31, kWave));
  return L;
}

__device__ __forceinline__ bool decode_tile256(const int32_t* __restrict__ offsets, int E, int ntn,
                                               int nsplit, bool pair_tails, const XcdList& L,
                                               int& e, int& beg, int& M, int& m0, int& nt,
                                               int& nt2, int& sp) {
  const int x = blockIdx.x & 7;
  int q = blockIdx.x >> 3;
  nt2 = -1;
  if ((ntn & 7) == 0) {
    if (q >= nsplit * L.n) return false;
    sp = q >= L.n ? 1 : 0;  // (nsplit <= 2)
    q -= sp * L.n;
    // the expert: the first whose tiles end past q
    const int lane = threadIdx.x & (kWave - 1);
    e = __popcll(__ballot(lane < E && L.il <= q));
    M = __builtin_amdgcn_readfirstlane(__shfl(L.ml, e, kWave));
    beg = __builtin_amdgcn_readfirstlane(__shfl(L.bl, e, kWave));
    q -= __builtin_amdgcn_readfirstlane(__shfl(L.il - L.cl, e, kWave));
    const int nnx = ntn >> 3;  // weight tiles of each XCD
    // the XCD's weight tiles in pairs (2g, 2g+1); an odd one left over last
    const int pairs = nnx >> 1;
    const int mt = (M + DT - 1) / DT;
    // small: the last m-tile holds at most DT/2 rows and is shared by the pair
    const bool small = pair_tails && pairs > 0 && mt > 0 && M - (mt - 1) * DT <= DT / 2;
    const int mf = small ? mt - 1 : mt;  // m-tiles a weight tile runs alone
    const int gsz = 2 * mf + (small ? 1 : 0);  // tiles of a pair's group
    if (q < pairs * gsz) {
      // group g: the shared last m-tile (if small), then the two weight
      // tiles' m-tiles alternately, so that the tiles reading either weight
      // tile run together
      const int g = q / gsz, r = q % gsz;
      if (small && r == 0) {
        m0 = mf * DT;
        nt = 2 * g * 8 + x;
        nt2 = nt + 8;
      } else {
        const int rr = small ? r - 1 : r;
        m0 = (rr >> 1) * DT;
        nt = (2 * g + (rr & 1)) * 8 + x;
      }
    } else {
      const int qq = q - pairs * gsz;
      m0 = (qq % mt) * DT;
      nt = (2 * pairs + qq / mt) * 8 + x;
    }
    return true;
  }
  int total = 0;
  for (int i = 0; i < E; ++i) total += ((offsets[i + 1] - offsets[i] + DT - 1) / DT) * ntn * nsplit;
  const int per = (total + 7) / 8;
  if (q >= per) return false;
  int Lq = x * per + q;
  if (Lq >= total) return false;
  for (int i = 0; i < E; ++i) {
    const int Mi = offsets[i + 1] - offsets[i];
    const int mt = (Mi + DT - 1) / DT;
    const int cnt = mt * ntn * nsplit;
    if (Lq < cnt) {
      e = i;
      beg = offsets[i];
      M = Mi;
      m0 = (Lq % mt) * DT;
      const int r = Lq / mt;
      nt = r % ntn;
      sp = r / ntn;
      return true;
    }
    Lq -= cnt;
  }
  return false;
}

// The down projection's K split, chosen by every workgroup from the expert
// counts (the same choice in all of them). With a split, every tile's longer
// first K part is listed before any second part, so the short second parts
// fill the last round over an XCD's CUs; the price is a second fixed cost
// per tile and a second float32 partial of y for the combine to read. The
// model: one XCD's 32 CUs take its n tiles (the list above) in order, each CU
// the next tile as soon as it is free (one workgroup per CU); every tile
// costs its K steps plus kFixSteps whatever its row count (a part-filled tile
// issues the loads of a full one, and those set its time: measured,
// part-filled and full tiles of the down projection take about as long); the
// combine's extra read costs `pen` K steps. It compares no split with first
// parts of 8/16 .. 13/16 of K (whole 4-step trips), one candidate per lane,
// and takes the fastest, no split on a tie; beyond 8 rounds of tiles per XCD
// it does not split. Measured at 4096 tokens, d = 4096, ffn = 14336 (down,
// us): k = 1: 625 unsplit, 530 / 497 / 530 / 555 with first parts of 8 / 11 /
// 12 / 13 sixteenths (the model picks 11); 16 experts: 985 unsplit, 907-914
// split at 11-13; 8x22B (d = 6144, 2048 tokens): 776 unsplit, 779-813 split
// (the model keeps it whole).
constexpr int kFixSteps = 12;  // start-up and epilogue of a tile, in K steps
constexpr int kXcdCUs = 32;    // compute units of one XCD

// Finish time of kXcdCUs CUs taking n tiles of cost a and then n of cost b
// (a, b > 0), each the next tile as soon as it is free. After the first
// parts, r = n % kXcdCUs CUs are at L + a and the others at L (L = (n /
// kXcdCUs) a); the second parts start at the n smallest of the times L + m b
// (each for the kXcdCUs - r lower CUs) and L + a + m b (each for the r upper
// ones), m = 0, 1, ...; the finish is the n-th smallest start plus b, or L + a
// if that is later. With a = alpha b + beta (0 <= beta < b), the starts up to
// L + a + m b number 32 (m + 1) + (32 - r) alpha, and those up to L + m b (m b
// >= a) number 32 (m + 1) - r (alpha + [beta > 0]).
__device__ __forceinline__ int two_part_makespan(int n, int a, int b) {
  const int L = (n / kXcdCUs) * a, r = n % kXcdCUs, nlo = kXcdCUs - r;
  int t = ((n + nlo - 1) / nlo - 1) * b;  // the n-th start if the lower CUs took all
  if (r > 0 && t >= a) {
    const int al = a / b, up = al + (a % b ? 1 : 0);
    const int mhi = max(0, (n - nlo * al + kXcdCUs - 1) / kXcdCUs - 1);
    const int mlo = max(up, (n + r * up + kXcdCUs - 1) / kXcdCUs - 1);
    t = min(a + mhi * b, mlo * b);
  }
  return L + max(t + b, r > 0 ? a : 0);
}

// steps of the first K part (a multiple of 4), or 0 for no split; n tiles of
// one K part per XCD
__device__ __forceinline__ int down_split_steps(int n, int nsteps, int pen) {
  if (n == 0 || n > 8 * kXcdCUs) return 0;
  // lane 0: no split; lane i = 1..6: a first part of i + 7 sixteenths. key =
  // finish time * 8 + lane, so the smallest key is the fastest, a tie going
  // to no split, then to the shorter first part
  const int lane = threadIdx.x & (kWave - 1);
  int key = 0x7fffffff;
  if (lane == 0) {
    key = (n + kXcdCUs - 1) / kXcdCUs * (nsteps + kFixSteps) * 8;
  } else if (lane <= 6) {
    const int s0 = (nsteps * (lane + 7) / 16) & ~3;
    if (s0 >= 4 && nsteps - s0 >= 4)
      key = (two_part_makespan(n, s0 + kFixSteps, nsteps - s0 + kFixSteps) + pen) * 8 + lane;
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) key = min(key, __shfl_xor(key, o, kWave));
  const int best = __builtin_amdgcn_readfirstlane(key) & 7;
  return best == 0 ? 0 : (nsteps * (best + 7) / 16) & ~3;
}

// GATE_UP: act = x [act_rows = T, K = d] bf16, wa/wb = w1/w3 [E, N = ffn, d],
// out = h [A, ffn] bf16, one K part; last m-tiles paired (fragment order).
// !GATE_UP: act = h [act_rows = A, K = ffn] bf16 in grouped order, wa = w2
// [E, N = d, ffn], out = part [nsplit][A][d] float32, the partial arrays
// pstride floats apart; with nsplit = 2 the K parts are [0, ksplit) and
// [ksplit, K). split: -1 = chosen here by down_split_steps (pen: the combine's
// extra read in K steps), 0 = one K part, > 0 = steps of the first part (a
// multiple of 4, at least 4 steps in each part). pair_tails: whether the tile
// list pairs last m-tiles of at most 128 rows (also what the split model
// counts; only fragment-order weights pair them, so both layouts choose the
// same split). ns_out (or null): receives nsplit, from workgroup 0. SCALED:
// sa/sb = row scales [E, N] of wa/wb.
template <bool GATE_UP, bool PACKED, bool SCALED>
__device__ __forceinline__ void dma_tile(const uint16_t* __restrict__ act, int64_t act_rows,
                                         const uint16_t* __restrict__ wa,
                                         const uint16_t* __restrict__ wb,
                                         const int32_t* __restrict__ offsets,
                                         const int32_t* __restrict__ sorted_asg, int K, int N,
                                         int E, int ktop, void* __restrict__ out, int ntn,
                                         int split, int pen, bool pair_tails,
                                         int32_t* __restrict__ ns_out, int64_t pstride,
                                         const float* __restrict__ sa,
                                         const float* __restrict__ sb) {
  // the tile list (row-major weights run every last m-tile on its own)
  const bool xcd = (ntn & 7) == 0;
  XcdList xl{0, 0, 0, 0, 0};
  if (xcd) xl = xcd_list(offsets, E, ntn, PACKED && pair_tails);
  int nsplit = 1, ksplit = K;
  if constexpr (!GATE_UP) {
    int s0 = split;
    if (split < 0) {
      // the split model counts the tiles as fragment order lists them, so
      // that both weight layouts choose the same split
      int n = xl.n;
      if (!PACKED && xcd && pair_tails) {
        const int lane = threadIdx.x & (kWave - 1);
        n = __builtin_amdgcn_readfirstlane(
            __shfl(prefix32(expert_tiles(xl.ml, ntn >> 3, true), lane), 31, kWave));
      }
      s0 = xcd ? down_split_steps(n, K / 32, pen) : 0;
    }
    if (s0 > 0) {
      nsplit = 2;
      ksplit = s0 * 32;
    }
    if (ns_out && blockIdx.x == 0 && threadIdx.x == 0) *ns_out = nsplit;
  }
  int e, beg, M, m0, nt, nt2, sp;
  if (!decode_tile256(offsets, E, ntn, nsplit, PACKED && pair_tails, xl, e, beg, M, m0, nt, nt2,
                      sp))
    return;

  // one array per buffer: distinct objects let the compiler see that a
  // fragment read does not depend on the loads in flight to other buffers
  // (fragment order: four K32 weight buffers; row-major: three K64 weight stages)
  constexpr int kWB012 = PACKED ? kWBufE : kTBufE;
  constexpr int kWB3 = PACKED ? kWBufE : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t wb0[kWB012];
  __shared__ __attribute__((aligned(1024))) uint16_t wb1[kWB012];
  __shared__ __attribute__((aligned(1024))) uint16_t wb2[kWB012];
  __shared__ __attribute__((aligned(1024))) uint16_t wb3[kWB3];
  __shared__ __attribute__((aligned(1024))) uint16_t tb0[kTBufE];
  __shared__ __attribute__((aligned(1024))) uint16_t tb1[kTBufE];
  // (fragment order only: the token stages of a paired tile)
  constexpr int kXB = PACKED ? kWBufE : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t xb0[kXB];
  __shared__ __attribute__((aligned(1024))) uint16_t xb1[kXB];
  auto wbufp = [&](auto bi) -> uint16_t* {
    constexpr int B = decltype(bi)::value;
    if constexpr (B == 0) return wb0;
    else if constexpr (B == 1) return wb1;
    else if constexpr (B == 2) return wb2;
    else return wb3;
  };
  auto tbufp = [&](auto bi) -> uint16_t* {
    constexpr int B = decltype(bi)::value;
    if constexpr (B == 0) return tb0;
    else return tb1;
  };
  // A paired tile (WIDE; fragment order only) computes the last m-tile, at
  // most 128 rows, of two weight tiles nt and nt2 of the same expert: wave
  // (wn, wm) takes 64 weight rows of tile wm ? nt2 : nt and the tile's 128
  // token rows, so each wave does what it does in a 256x256 tile. A step's 32
  // weight fragments (two 16 KiB halves) sit in weight buffer b: b = 0 in
  // tb0, b = 1 in wb0 and wb1, b = 2 in tb1, b = 3 in wb2 and wb3; the two
  // 16 KiB token stages in xb0 and xb1. Each LDS array still serves one
  // buffer only, so no fragment read shares an array with a load in flight.
  auto body = [&](auto widec) {
  constexpr bool WIDE = decltype(widec)::value;
  // (the half is a compile-time constant: a pointer chosen at run time
  // between two arrays would hide which array a fragment read touches)
  auto wbw = [&](auto bi, auto hc) -> uint16_t* {
    constexpr int B = decltype(bi)::value;
    constexpr int H = decltype(hc)::value;
    if constexpr (B == 0) return tb0 + H * kWBufE;
    else if constexpr (B == 1) return H ? wb1 : wb0;
    else if constexpr (B == 2) return tb1 + H * kWBufE;
    else return H ? wb3 : wb2;
  };
  auto tsp = [&](auto bi) -> uint16_t* {
    constexpr int B = decltype(bi)::value;
    if constexpr (WIDE) {
      if constexpr (B == 0) return xb0;
      else return xb1;
    } else {
      return tbufp(bi);
    }
  };
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = w & 3, wm = w >> 2;
  const int fr = lane & 15, fg = lane >> 4;
  // this tile's K range: [k0, k0 + Kc)
  const int k0 = (GATE_UP || sp == 0) ? 0 : ksplit;
  const int Kc = (GATE_UP || nsplit == 1) ? K : (sp == 0 ? ksplit : K - ksplit);
  // LDS weight fragment f (of 16) is wave wn = f >> 2's tile f & 3. Gate/up:
  // w1 rows for f & 3 < 2, else w3 rows, nt*128 + (f >> 2)*32 + (f & 1)*16;
  // wave w loads fragments 2w, 2w+1 (all w1 for even w, all w3 for odd w).
  // Down: w2 rows nt*256 + 16 f; wave w loads fragments 2w, 2w+1.
  const size_t wslice = static_cast<size_t>(N) * K;  // elements of one expert matrix
  const uint16_t* wsrc = (GATE_UP && (w & 1)) ? wb : wa;
  const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(wsrc + e * wslice), 0, static_cast<int>(wslice * 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(act), 0, static_cast<int>(act_rows * K * 2), kRsrcWord3);
  int aoff[2][2];  // fragment order: byte offsets of step 0 (wave-uniform), [half][q]
  // row-major: per-lane byte offsets of stage 0 for the loads q = 0, 2 and
  // q = 1, 3 (rows placed as the token rows below; load q reads 8q rows
  // further, a wave-uniform offset, and the swizzle slot depends on q % 2)
  int woff[2];
  if constexpr (PACKED) {
#pragma unroll
    for (int hh = 0; hh < (WIDE ? 2 : 1); ++hh) {
      const int ntt = hh ? nt2 : nt;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int row =
            GATE_UP ? ntt * 128 + (w >> 1) * 32 + q * 16 : ntt * 256 + (2 * w + q) * 16;
        aoff[hh][q] =
            __builtin_amdgcn_readfirstlane(static_cast<int>(wofs<true>(0, row, k0, N, K) * 2));
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = 32 * w + 8 * q + (lane >> 3);  // LDS row = 16 * fragment + fragment row
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int row = GATE_UP ? nt * 128 + (w >> 1) * 32 + 8 * q + (lane >> 3) : nt * 256 + r;
      woff[q] = (row * K + k0 + c * 8) * 2;
    }
  }
  // token loads: wave w moves tile rows 32w .. 32w+31, 8 rows x 128 B per load; lane l puts row
  // 32w + 8q + l/8, LDS slot l%8, which holds 16-byte chunk (l%8) ^ ((row/2) % 8) of the K64 stage
  // (paired tile: 128 rows, wave w rows 16w .. 16w+15, two loads)
  constexpr int kTQ = WIDE ? 2 : 4;   // token loads of a wave per stage
  constexpr int kTR = 8 * kTQ;        // token rows of a wave
  int toff[kTQ];
#pragma unroll
  for (int q = 0; q < kTQ; ++q) {
    const int r = kTR * w + 8 * q + (lane >> 3);
    const int mm = min(m0 + r, M - 1);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int src = GATE_UP ? sorted_asg[beg + mm] / ktop : beg + mm;
    toff[q] = (src * K + k0 + c * 8) * 2;
  }
  const int lane16 = lane * 16;
  const int nsteps = Kc / 32;      // a multiple of 4
  const int last = nsteps - 1;
  const int last_stage = nsteps / 2 - 1;
  auto load_w = [&](uint16_t* L, int q, int t) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr)(L + (2 * w + q) * kFragE), 16, lane16,
                                             aoff[0][q] + t * (kFragE * 2), 0, 0);
  };
  // paired tile: both fragments of this wave in half hh of weight buffer bi
  auto load_w2 = [&](auto bi, auto hc, int t) {
    constexpr int H = decltype(hc)::value;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr)(wbw(bi, hc) + (2 * w + q) * kFragE),
                                               16, lane16, aoff[H][q] + t * (kFragE * 2), 0, 0);
  };
  auto load_x = [&](uint16_t* L, int q, int s) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, (lds_ptr)(L + (kTR * w + 8 * q) * 64), 16,
                                             toff[q], s * 128, 0, 0);
  };
  auto load_ws = [&](uint16_t* L, int q, int s) {  // row-major weights, K64 stage s
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, (lds_ptr)(L + (32 * w + 8 * q) * 64), 16,
                                             woff[q & 1], s * 128 + (q >> 1) * 16 * K * 2, 0, 0);
  };
  // prologue: the loads steps -4 .. -1 would have issued in the steady state
  // (weights of steps 0-3, token stages 0-1; odd steps tokens first), so the
  // loop's wait counts hold from its first step
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // (row-major weights: weight stages 0-2 and token stages 0-1, in the order
  // odd steps issue them, tokens of stage s with weights of stage s+1)
  if constexpr (WIDE) {
    load_w2(I0{}, I0{}, 0); load_w2(I0{}, I1{}, 0);
    load_x(tsp(I0{}), 0, 0); load_x(tsp(I0{}), 1, 0);
    load_w2(I1{}, I0{}, min(1, last)); load_w2(I1{}, I1{}, min(1, last));
    load_w2(I2{}, I0{}, min(2, last)); load_w2(I2{}, I1{}, min(2, last));
    load_x(tsp(I1{}), 0, min(1, last_stage)); load_x(tsp(I1{}), 1, min(1, last_stage));
    load_w2(I3{}, I0{}, min(3, last)); load_w2(I3{}, I1{}, min(3, last));
  } else if constexpr (PACKED) {
    load_w(wbufp(I0{}), 0, 0); load_w(wbufp(I0{}), 1, 0);
    load_x(tbufp(I0{}), 0, 0); load_x(tbufp(I0{}), 1, 0); load_x(tbufp(I0{}), 2, 0); load_x(tbufp(I0{}), 3, 0);
    load_w(wbufp(I1{}), 0, min(1, last)); load_w(wbufp(I1{}), 1, min(1, last));
    load_w(wbufp(I2{}), 0, min(2, last)); load_w(wbufp(I2{}), 1, min(2, last));
    load_x(tbufp(I1{}), 0, min(1, last_stage)); load_x(tbufp(I1{}), 1, min(1, last_stage));
    load_x(tbufp(I1{}), 2, min(1, last_stage)); load_x(tbufp(I1{}), 3, min(1, last_stage));
    load_w(wbufp(I3{}), 0, min(3, last)); load_w(wbufp(I3{}), 1, min(3, last));
  } else {
    const int s1 = min(1, last_stage), s2 = min(2, last_stage);
    load_ws(wbufp(I0{}), 0, 0); load_ws(wbufp(I0{}), 1, 0); load_ws(wbufp(I0{}), 2, 0); load_ws(wbufp(I0{}), 3, 0);
    load_x(tbufp(I0{}), 0, 0); load_x(tbufp(I0{}), 1, 0); load_x(tbufp(I0{}), 2, 0); load_x(tbufp(I0{}), 3, 0);
    load_ws(wbufp(I1{}), 0, s1); load_ws(wbufp(I1{}), 1, s1); load_ws(wbufp(I1{}), 2, s1); load_ws(wbufp(I1{}), 3, s1);
    load_x(tbufp(I1{}), 0, s1); load_x(tbufp(I1{}), 1, s1); load_x(tbufp(I1{}), 2, s1); load_x(tbufp(I1{}), 3, s1);
    load_ws(wbufp(I2{}), 0, s2); load_ws(wbufp(I2{}), 1, s2); load_ws(wbufp(I2{}), 2, s2); load_ws(wbufp(I2{}), 3, s2);
  }

  // fragments of this wave's token tiles that hold a row, rounded up to even
  const int valid = M - m0 - (WIDE ? 0 : wm * 128);
  const int jv = valid >= 128 ? 8 : valid <= 0 ? 0 : (((valid + 15) >> 4) + 1) & ~1;
  // token fragment reads: row (wm*128 + 16j + fr), chunk 4*half + fg, swizzled slot
  const int trow = ((WIDE ? 0 : wm * 128) + fr) * 64;
  const int tcol0 = ((fg) ^ ((fr >> 1) & 7)) * 8;
  const int tcol1 = ((4 + fg) ^ ((fr >> 1) & 7)) * 8;
  // row-major weight fragment reads: row (wn*64 + 16k + fr), same chunks and slots
  const int wrow = (wn * 64 + fr) * 64;

  // (WMC: the wave's wm as a constant, for the paired tile's weight reads)
  auto run = [&](auto jvc, auto wmc) {
    constexpr int JV = decltype(jvc)::value;
    constexpr int WMC = decltype(wmc)::value;
    u32x4 fa[2][4], fb[2][8];
    f32x4 acc[4][JV > 0 ? JV : 1];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JV; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fragment k of a step into register set si: k < 4 the wave's weight tile
    // k (weight buffer wi), k >= 4 its token tile k - 4 (token buffer ti, half hh)
    auto rd = [&](auto wi, auto ti, auto hh, auto si, int k) {
      constexpr int S = decltype(si)::value;
      constexpr int HH = decltype(hh)::value;
      if (k < 4) {
        if constexpr (WIDE)
          fa[S][k] = *reinterpret_cast<const u32x4*>(wbw(wi, wmc) + (wn * 4 + k) * kFragE + lane * 8);
        else if constexpr (PACKED)
          fa[S][k] = *reinterpret_cast<const u32x4*>(wbufp(wi) + (wn * 4 + k) * kFragE + lane * 8);
        else
          fa[S][k] = *reinterpret_cast<const u32x4*>(wbufp(wi) + wrow + k * 16 * 64 + (HH ? tcol1 : tcol0));
      } else if (k - 4 < JV) {
        const uint16_t* TL = tsp(ti);
        fb[S][k - 4] = *reinterpret_cast<const u32x4*>(TL + trow + (k - 4) * 16 * 64 + (HH ? tcol1 : tcol0));
      }
    };
    // weights of step 0 and token stage 0 (row-major: stage 0 of both)
    // (paired tile: 14, the prologue's later 4 + 4 + 2 + 4 loads)
    __builtin_amdgcn_s_waitcnt(vmcnt_le(WIDE ? 14 : PACKED ? 10 : 12));
    lds_barrier();
#pragma unroll
    for (int k = 0; k < 12; ++k) rd(I0{}, I0{}, I0{}, I0{}, k);

    int t0 = 0;
    auto step = [&](auto tm) {
      // step t = t0 + T: weights in wbuf T (row-major: wbuf (T/2) % 3), tokens
      // in tbuf T/2 half T%2 (t0 % 4 == 0; row-major: t0 % 12 == 0)
      constexpr int T = decltype(tm)::value;
      constexpr int CUR = T & 1, NXT = CUR ^ 1;
      using WN = std::integral_constant<int, PACKED ? (T + 1) & 3 : ((T + 1) >> 1) % 3>;
      using TN = std::integral_constant<int, ((T + 1) >> 1) & 1>;
      using HN = std::integral_constant<int, (T + 1) & 1>;
      const int t = t0 + T;
      // own loads of step t+1 done: weights (issued in step t-3) and its token
      // stage (issued in step t-2 for odd t, t-3 for even t; counted from the
      // issue order above); the barrier publishes step t+1 and frees the
      // buffers step t was read from (it is in registers)
      // (row-major weights: step t+1 of an odd step t is stage (t+1)/2, whose
      // tokens went out in step t-2 before the weights of stage (t+3)/2 and
      // whose weights in step t-4; even steps need nothing new)
      // (paired tile: 4 weight loads a step and 2 token loads in odd steps,
      // so 8 and 10)
      __builtin_amdgcn_s_waitcnt(
          vmcnt_le((T & 1) ? (WIDE ? 8 : 4) : (WIDE ? 10 : PACKED ? 8 : 12)));
      lds_barrier();
      const int tw = min(t + 4, last);
      const int ts = min((t + 3) >> 1, last_stage);
      const int ts5 = min((t + 5) >> 1, last_stage);
      unrolled([&](auto gm) {
        constexpr int g = decltype(gm)::value;
        constexpr int i = g >> 1, j0 = (g & 1) * 4;
        unrolled([&](auto jm) {
          constexpr int j = j0 + decltype(jm)::value;
          if constexpr (j < JV) acc[i][j] = mfma16x16x32(fa[CUR][i], fb[CUR][j], acc[i][j]);
        }, std::make_integer_sequence<int, 4>{});
        if constexpr (g < 4) {
          // next step's fragments in the order it uses them: tokens 0-3,
          // weight 0, tokens 4-7, weights 1-3
          constexpr int order[12] = {4, 5, 6, 7, 0, 8, 9, 10, 11, 1, 2, 3};
          unrolled([&](auto rm) {
            rd(WN{}, TN{}, HN{}, std::integral_constant<int, NXT>{}, order[3 * g + decltype(rm)::value]);
          }, std::make_integer_sequence<int, 3>{});
          if constexpr (WIDE) {
            // odd steps: tokens of stage (t+3)/2, then both halves of step
            // t+4's weights; even steps: both halves of step t+4's weights
            using TB = std::integral_constant<int, ((T + 3) >> 1) & 1>;
            if constexpr (T & 1) {
              if constexpr (g == 0) { load_x(tsp(TB{}), 0, ts); load_x(tsp(TB{}), 1, ts); }
              else if constexpr (g < 3) load_w2(tm, std::integral_constant<int, g - 1>{}, tw);
            } else if constexpr (g < 2) {
              load_w2(tm, std::integral_constant<int, g>{}, tw);
            }
          } else if constexpr (T & 1) {
            // tokens of stage (t+3)/2 into the buffer stage (t-1)/2 has left,
            // then the weights of step t+4 (row-major: of stage (t+5)/2, into
            // the buffer stage (t-1)/2 has left)
            using TB = std::integral_constant<int, ((T + 3) >> 1) & 1>;
            using WB = std::integral_constant<int, ((T + 5) >> 1) % 3>;
            if constexpr (g < 2) { load_x(tbufp(TB{}), 2 * g, ts); load_x(tbufp(TB{}), 2 * g + 1, ts); }
            else if constexpr (PACKED) load_w(wbufp(tm), g - 2, tw);
            else { load_ws(wbufp(WB{}), 2 * g - 4, ts5); load_ws(wbufp(WB{}), 2 * g - 3, ts5); }
          } else if constexpr (PACKED) {
            if constexpr (g < 2) load_w(wbufp(tm), g, tw);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }, std::make_integer_sequence<int, 8>{});
    };
    // unrolled over a whole buffer cycle so that every buffer index is a
    // constant: 4 steps, or 12 with row-major weights (3 weight stages x 2
    // token stages), then the remaining 4 or 8 steps with the first cycle's
    // indices (the remainder starts at a multiple of 12)
    constexpr int UNR = PACKED ? 4 : 12;
    for (; t0 + UNR <= nsteps; t0 += UNR) unrolled(step, std::make_integer_sequence<int, UNR>{});
    if constexpr (!PACKED) {
      if (t0 < nsteps) {
        unrolled(step, std::make_integer_sequence<int, 4>{});
        if (t0 + 4 < nsteps)
          unrolled([&](auto i) { step(std::integral_constant<int, decltype(i)::value + 4>{}); },
                   std::make_integer_sequence<int, 4>{});
      }
    }
    // epilogue: lane holds token column fr of each 16x16 tile and weight rows
    // 4*fg .. 4*fg+3 of it; gate/up: gate in tiles 0-1, up in tiles 2-3. An
    // empty asm with VGPR constraints (no instruction) fixes the accumulators'
    // register class for the allocator.
    // (SCALED: the row scales of the lane's 4 rows of a weight tile, read
    // where they are used; cache hits after the first token tile)
    const int ntw = WIDE && WMC ? nt2 : nt;  // the wave's weight tile
    const float* rsa = SCALED ? sa + static_cast<size_t>(e) * N : nullptr;
    const float* rsb = SCALED ? sb + static_cast<size_t>(e) * N : nullptr;
    if constexpr (GATE_UP) {
      // h through LDS, then whole rows to global memory, for both weight
      // layouts: each store instruction writes 1 KiB of whole 128-byte lines
      // instead of 16 pieces of 32 bytes (8x7B prefill, fragment order: 2.378
      // -> 2.367 ms per layer).
      // tb0 and tb1 are free once every load has landed (the last steps'
      // loads only repeat the last step's data: they are waited for here) and
      // every wave is past its last fragment read (the barrier). Staged tile:
      // 256 rows x 128 columns (paired: 128 x 256), 16-byte chunk c of row r
      // at slot c ^ (r % 16) of the row, the first half of the rows in tb0,
      // the rest in tb1.
      constexpr int kCh = WIDE ? 32 : 16;  // 16-byte chunks per staged row
      constexpr int kRowsHalf = WIDE ? 64 : 128;
      auto slot = [&](int r, int c) -> uint16_t* {
        uint16_t* b = r < kRowsHalf ? tb0 : tb1;
        return b + ((r % kRowsHalf) * kCh + (c ^ (r & 15))) * 8;
      };
      __builtin_amdgcn_s_waitcnt(vmcnt_le(0));
      lds_barrier();
#pragma unroll
      for (int j = 0; j < JV; ++j) {
        const int r = (WIDE ? 0 : wm * 128) + j * 16 + fr;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int n = ntw * 128 + wn * 32 + i * 16 + 4 * fg;
          const int col = (WIDE ? WMC * 128 : 0) + wn * 32 + i * 16 + 4 * fg;
          f32x4 gt = acc[i][j];
          f32x4 up = acc[i + 2][j];
          asm volatile("" : "+v"(gt), "+v"(up));
          if constexpr (SCALED) {
            gt *= *reinterpret_cast<const f32x4*>(rsa + n);
            up *= *reinterpret_cast<const f32x4*>(rsb + n);
          }
          uint2 v;
          v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
          v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
          *reinterpret_cast<uint2*>(slot(r, col >> 3) + (col & 7)) = v;
        }
      }
      lds_barrier();
      // wave w stores rows w * R/8 .. (R = 256, paired 128), 64 / kCh rows
      // per instruction; rows past the expert's end are not stored
      constexpr int kRowsW = (WIDE ? 128 : 256) / 8, kPer = 64 / kCh;
#pragma unroll
      for (int it = 0; it < kRowsW / kPer; ++it) {
        const int r = w * kRowsW + it * kPer + lane / kCh;
        const int c = lane % kCh;
        if (m0 + r < M) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(slot(r, c));
          const int ntc = WIDE ? (c < 16 ? nt : nt2) : nt;
          *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) +
                                    static_cast<size_t>(beg + m0 + r) * N + ntc * 128 +
                                    (c & 15) * 8) = v;
        }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < JV; ++j) {
      const int m = m0 + (WIDE ? 0 : wm * 128) + j * 16 + fr;
      if (m >= M) continue;
      if constexpr (GATE_UP) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int n = ntw * 128 + wn * 32 + i * 16 + 4 * fg;
          f32x4 gt = acc[i][j];
          f32x4 up = acc[i + 2][j];
          asm volatile("" : "+v"(gt), "+v"(up));
          if constexpr (SCALED) {
            gt *= *reinterpret_cast<const f32x4*>(rsa + n);
            up *= *reinterpret_cast<const f32x4*>(rsb + n);
          }
          uint2 v;
          v.x = pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]);
          v.y = pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + static_cast<size_t>(beg + m) * N +
                                    n) = v;
        }
      } else {
        float* y = static_cast<float*>(out) + sp * pstride + static_cast<size_t>(beg + m) * N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 v = acc[i][j];
          asm volatile("" : "+v"(v));
          if constexpr (SCALED)
            v *= *reinterpret_cast<const f32x4*>(rsa + ntw * 256 + wn * 64 + i * 16 + 4 * fg);
          *reinterpret_cast<f32x4*>(y + ntw * 256 + wn * 64 + i * 16 + 4 * fg) = v;
        }
      }
    }
  };
  auto run_wm = [&](auto jvc) {
    if constexpr (WIDE) {
      if (wm) run(jvc, I1{});
      else run(jvc, I0{});
    } else {
      run(jvc, I0{});
    }
  };
  switch (jv) {
    case 8: run_wm(std::integral_constant<int, 8>{}); break;
    case 6: run_wm(std::integral_constant<int, 6>{}); break;
    case 4: run_wm(std::integral_constant<int, 4>{}); break;
    case 2: run_wm(std::integral_constant<int, 2>{}); break;
    default: run_wm(std::integral_constant<int, 0>{}); break;
  }
  };
  if constexpr (PACKED) {
    if (nt2 >= 0) body(std::true_type{});
    else body(std::false_type{});
  } else {
    body(std::false_type{});
  }
}

// x [T, d] bf16, w1/w3 [E, ffn, d] (fragment order or row-major), h [A, ffn] bf16
template <bool PACKED, bool SCALED>
__global__ __launch_bounds__(kDmaThreads, 1) void gate_up_dma_kernel(
    const uint16_t* __restrict__ x, int64_t T, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ w3, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_asg, int d, int ffn, int E, int ktop,
    uint16_t* __restrict__ h, int ntn, const float* __restrict__ s1, const float* __restrict__ s3) {
  dma_tile<true, PACKED, SCALED>(x, T, w1, w3, offsets, sorted_asg, d, ffn, E, ktop, h, ntn, 0, 0,
                                 true, nullptr, 0, s1, s3);
}

// h [A, ffn] bf16 grouped, w2 [E, d, ffn] (fragment order or row-major), part [nsplit, A, d] f32
template <bool PACKED, bool SCALED>
__global__ __launch_bounds__(kDmaThreads, 1) void down_dma_kernel(
    const uint16_t* __restrict__ h, int64_t A, const uint16_t* __restrict__ w2,
    const int32_t* __restrict__ offsets, int d, int ffn, int E, float* __restrict__ part, int ntn,
    int split, int pen, int pair_tails, int32_t* __restrict__ ns_out,
    const float* __restrict__ s2) {
  dma_tile<false, PACKED, SCALED>(h, A, w2, w2, offsets, nullptr, ffn, d, E, 1, part, ntn, split,
                                  pen, pair_tails != 0, ns_out, A * d, s2, s2);
}

constexpr int64_t kMax31 = (int64_t(1) << 31) - 1;

}  // namespace

bool dma_gate_up_ok(int64_t A, int k, int d, int ffn, int E) {
  if (d % 128 != 0 || ffn % 128 != 0) return false;
  // every tile costs a full pass over its weight rows whatever its token
  // count; measured at the 8x7B shape, these tiles beat the 128-row ones from
  // 128 rows per expert on average (T = 512: 399 vs 498 us) but not at 64
  // (368 vs 355 us)
  if (A < static_cast<int64_t>(DT / 2) * E) return false;
  // byte offsets inside the buffer descriptors are 31-bit
  return static_cast<int64_t>(ffn) * d * 2 <= kMax31 && (A / k) * d * 2 <= kMax31;
}

hipError_t launch_gate_up_dma(bool packed, const uint16_t* x, const uint16_t* w1,
                              const uint16_t* w3, const int32_t* offsets,
                              const int32_t* sorted_asg, int64_t A, int d, int ffn, int E, int k,
                              uint16_t* h, hipStream_t s, const float* s1, const float* s3) {
  const int ntn = ffn / 128;
  const int64_t tiles = ((A + DT - 1) / DT + E) * ntn;  // upper bound
  const dim3 grid(static_cast<unsigned>((tiles + 7) / 8 * 8));
  if (s1 && !packed) return hipErrorInvalidValue;  // row scales come with fragment order only
  if (s1)
    hipLaunchKernelGGL((gate_up_dma_kernel<true, true>), grid, dim3(kDmaThreads), 0, s, x, A / k,
                       w1, w3, offsets, sorted_asg, d, ffn, E, k, h, ntn, s1, s3);
  else if (packed)
    hipLaunchKernelGGL((gate_up_dma_kernel<true, false>), grid, dim3(kDmaThreads), 0, s, x, A / k,
                       w1, w3, offsets, sorted_asg, d, ffn, E, k, h, ntn, s1, s3);
  else
    hipLaunchKernelGGL((gate_up_dma_kernel<false, false>), grid, dim3(kDmaThreads), 0, s, x, A / k,
                       w1, w3, offsets, sorted_asg, d, ffn, E, k, h, ntn, s1, s3);
  return hipGetLastError();
}

bool dma_down_ok(int64_t A, int d, int ffn, int E) {
  if (d % 256 != 0 || ffn % 128 != 0) return false;
  // (down: from 256 rows per expert; at 128 the 128-row tiles were 6% faster)
  if (A < static_cast<int64_t>(DT) * E) return false;
  return static_cast<int64_t>(ffn) * d * 2 <= kMax31 && A * ffn * 2 <= kMax31;
}

// The most K parts the kernel may choose (the workspace holds that many
// partial arrays of y): 2 where the device's choice may split, i.e. weight
// tiles in multiples of 8, at least 8 K steps, and an XCD's tiles possibly
// within 8 rounds of its CUs (a lower bound of their count: every expert's
// rows in whole m-tiles, less one per pair of weight tiles for its last).
int dma_down_splits(int64_t A, int d, int ffn, int E) {
  if (!dma_down_ok(A, d, ffn, E) || (d / 256) % 8 != 0 || ffn / 32 < 8) return 1;
  const int64_t nnx = d / 2048;
  return nnx * (A / DT - (E + 1) / 2) <= 8 * kXcdCUs ? 2 : 1;
}

hipError_t launch_down_dma(bool packed, const uint16_t* h, const uint16_t* w2,
                           const int32_t* offsets, int64_t A, int d, int ffn, int E,
                           int max_split, float* part, hipStream_t s, const float* s2,
                           DownSplit ds) {
  const int split_opt = ds.opt;
  int32_t* ns_out = ds.word;
  const int ntn = d / 256;
  const int nsteps = ffn / 32;
  if (max_split != 1 && max_split != 2) return hipErrorInvalidValue;
  const int64_t tiles = ((A + DT - 1) / DT + E) * ntn * max_split;  // upper bound
  const dim3 grid(static_cast<unsigned>((tiles + 7) / 8 * 8));
  // split: -1 chosen on the device, 0 none, > 0 a caller's first part of
  // split_opt sixteenths of K (whole 4-step trips, at least 4 steps each)
  int split = 0;
  if (max_split == 2) {
    if (split_opt == 0) {
      split = -1;
    } else if (split_opt >= 8 && split_opt <= 13) {
      const int s0 = (nsteps * split_opt / 16) & ~3;
      split = (s0 >= 4 && nsteps - s0 >= 4) ? s0 : 0;
    }
  }
  const int pair = A <= static_cast<int64_t>(2 * DT) * E;
  // the combine's read of the second partial (A*d*4 bytes at about 5 TB/s) in
  // tile K steps (about 0.85 us each at the measured MFMA rate)
  const int pen = static_cast<int>((A * d) >> 20);
  if (s2 && !packed) return hipErrorInvalidValue;  // row scales come with fragment order only
  if (s2)
    hipLaunchKernelGGL((down_dma_kernel<true, true>), grid, dim3(kDmaThreads), 0, s, h, A, w2,
                       offsets, d, ffn, E, part, ntn, split, pen, pair, ns_out, s2);
  else if (packed)
    hipLaunchKernelGGL((down_dma_kernel<true, false>), grid, dim3(kDmaThreads), 0, s, h, A, w2,
                       offsets, d, ffn, E, part, ntn, split, pen, pair, ns_out, s2);
  else
    hipLaunchKernelGGL((down_dma_kernel<false, false>), grid, dim3(kDmaThreads), 0, s, h, A, w2,
                       offsets, d, ffn, E, part, ntn, split, pen, pair, ns_out, s2);
  return hipGetLastError();
}

}  // namespace moe
