// Large-M product of MXFP4 weights with MXFP8 activations on gfx950's
// MX-scaled matrix cores.
//
// At M = 1 the expert path is a bandwidth-bound GEMV; grouping the active
// experts into a GEMM is the lever the gpt-oss page names and leaves untried
// ("Sovereign gpt-oss-20B (MXFP4) on Apple Silicon", section 5), and the q4
// page puts fp8 / grouped-expert GEMM beyond its single-stream floor
// ("Amortizing the per-token host-sync setup tax ...", section 5).  With many
// tokens per weight byte (prefill) the product becomes a dense contraction,
// so it runs on V_MFMA_SCALE_F32_32X32X64_F8F6F4: A = 32 weight rows x 64 K
// in FP4 E2M1, B = 64 K x 32 tokens in FP8 E4M3, one E8M0 scale per operand
// row and 32-element K block, fp32 accumulation.  The MXFP4 weights are
// multiplied as stored (PLAIN layout, no repacking); the activations are
// first quantized to MXFP8 (OCP MX v1.0 conversion) by mxfp8_quant_kernel.
//
// Operand lane layout of the instruction, as measured on the device (one
// wavefront, lane l, j = l % 32, h = l / 32):
//   A (FP4, 4 VGPRs): row j, K elements 32h .. 32h+31 in nibble order (low
//     nibble first) - exactly 16 consecutive bytes of a PLAIN code row; the
//     lane's scale byte is the E8M0 of that 32-element block.
//   B (FP8, 8 VGPRs): column j; bytes 0..15 are K 16h .. 16h+15, bytes
//     16..31 are K 32+16h .. 32+16h+15; the lane's scale byte is the E8M0 of
//     K block h (K 0..31 or 32..63) of column j.
//   D (16 fp32): register r holds row 8(r/4) + 4h + (r%4), column j.
// The instruction adds its 64 products at reduced internal precision
// (measured: up to ~1e-4 of the sum of |products| per instruction), so the
// product is compared with the oracle under a tolerance relative to
// sum |W| |xq|, not bit for bit.
#include "bdg_device.hpp"
#include "bdg_host.hpp"

namespace bdg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kQuantThreads = 256;

// fp32 -> FP8 E4M3 code: round to nearest, ties to even, saturating at 448.
// Sign kept (so -0.0 and negative values that round to 0 give 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t s = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t c;
  if (a >= 0x43E00000u) {                   // |v| >= 448
    c = 0x7Eu;
  } else if (a >= 0x3C800000u) {            // 2^-6 <= |v| < 448: normal
    // keep 3 mantissa bits: round the 20 dropped bits half to even, then
    // rebias the exponent from 127 to 7 (a carry moves to the next binade)
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    c = r - (120u << 3);
    if (c > 0x7Eu) c = 0x7Eu;
  } else {                                  // subnormal: multiples of 2^-9
    c = (uint32_t)rintf(__uint_as_float(a) * 512.0f);   // exact scaling; 8 = smallest normal
  }
  return s | c;
}

// One 32-element block per 8 threads, 4 elements per thread.
__global__ void __launch_bounds__(kQuantThreads)
mxfp8_quant_kernel(const void* __restrict__ x, int x_bf16, int64_t n_elems, uint8_t* __restrict__ codes,
                   uint8_t* __restrict__ scales) {
  const int64_t e0 = ((int64_t)blockIdx.x * kQuantThreads + threadIdx.x) * 4;
  const bool ok = e0 < n_elems;
  const int64_t ec = ok ? e0 : n_elems - 4;   // in bounds; results unused
  float v[4];
  if (x_bf16) {
    const uint2 b = ldg_u64(reinterpret_cast<const uint16_t*>(x) + ec);
    v[0] = bf16_to_f32((uint16_t)(b.x & 0xFFFFu));
    v[1] = bf16_to_f32((uint16_t)(b.x >> 16));
    v[2] = bf16_to_f32((uint16_t)(b.y & 0xFFFFu));
    v[3] = bf16_to_f32((uint16_t)(b.y >> 16));
  } else {
    const float4 f = ldg_f4(reinterpret_cast<const float*>(x) + ec);
    v[0] = f.x;
    v[1] = f.y;
    v[2] = f.z;
    v[3] = f.w;
  }
  // block maximum of |v| as bits (non-negative floats order as integers);
  // any NaN or infinity makes the block non-finite
  uint32_t amax = 0, bad = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = __float_as_uint(v[i]) & 0x7FFFFFFFu;
    bad |= a >= 0x7F800000u ? 1u : 0u;
    amax = max(amax, a);
  }
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    amax = max(amax, (uint32_t)__shfl_xor((int)amax, d));
    bad |= (uint32_t)__shfl_xor((int)bad, d);
  }
  // X = floor(log2 amax) - 8, clamped to >= -127 (amax = 0 or subnormal)
  const int eb = (int)(amax >> 23);            // biased exponent of amax
  int X = amax == 0 ? -127 : eb - 127 - 8;
  X = X < -127 ? -127 : X;
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X, X in [-127, 119]
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) word |= (bad ? 0x7Fu : f32_to_e4m3(v[i] * inv)) << (8 * i);
  if (ok) {
    *reinterpret_cast<uint32_t*>(codes + e0) = word;
    if ((threadIdx.x & 7) == 0) scales[e0 >> 5] = (uint8_t)(bad ? 255 : X + 127);
  }
}

constexpr int kBN = 256;            // weight rows per block
constexpr int kBK = 128;            // K per stage: two 64-deep MFMA steps, four 32-blocks
constexpr int kTA = 2;              // 32-row MFMA tiles per wave
constexpr int kRowGroups = kBN / (32 * kTA);   // 4 waves along the rows
constexpr int kNB = 1;              // 32-token MFMA tiles per wave

// The operands of one K stage are copied from global memory straight into
// LDS (global_load_lds: each lane of a wave sends its 16 - or 4 - bytes to
// the next slot of an LDS chunk, so nothing passes through VGPRs).  Three
// stages form a ring: the copies run two stages ahead of the MFMAs.  Each
// operand row is kept whole - A row r: its 4 pieces (32-blocks of the stage)
// in 16-byte slots 4r .. 4r+3; B token t: its 8 pieces (16 K each) in slots
// 8t .. 8t+7 - with the pieces XOR-permuted by the row, so that the 8 and
// the 16 lanes of one LDS pass of the MFMA operand reads (one piece of 8 or
// 16 consecutive rows) fall in distinct bank groups; the copy lanes fetch
// the matching global piece, so the permutation costs nothing.
//
// Scale bytes come stage-major (mx_stage_scales_kernel): word [s][row]
// holds the row's 4 E8M0 bytes of stage s (byte q = K block 4 s + q), so
// one stage's scales of a block's 256 weight rows are 1 KB in a row - 8
// cache lines - where the [row][K / 32] layout scatters them over ~180.
//
// Block shapes, by TM = tokens per block: 64 (8 waves, 4 row groups x 2
// token groups, a 76 KB ring: two blocks share a CU) or 128 (16 waves, a
// 100 KB ring: one block per CU, half the weight bytes per product).  A
// wave holds kTA = 2 row tiles and one token tile, so either shape runs 4
// waves per SIMD in under 128 VGPRs.
template <int TM>
struct MxShape {
  static_assert(TM == 64 || TM == 128, "64 or 128 tokens per block");
  static constexpr int kBM = TM;
  static constexpr int kWaves = kRowGroups * TM / 32;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kSlotsA = kBN * 4;              // 16-byte slots of A per stage (16 KB)
  static constexpr int kSlotsB = TM * 8;               // of B (8 or 16 KB)
  static constexpr int kDmaA = kSlotsA / 64 / kWaves;  // A chunks per wave and stage (2 or 1)
  static constexpr int kDmaB = kSlotsB / 64 / kWaves;  // B chunks per wave and stage (1)
  static constexpr int kDmaPerStage = kDmaA + kDmaB + 1;   // + one chunk of scale words
};

__device__ __forceinline__ int a_slot(int r, int q) { return 4 * r + (q ^ (((r >> 1) ^ (r >> 3)) & 3)); }
__device__ __forceinline__ int b_slot(int t, int p) { return 8 * t + (p ^ ((t ^ (t >> 3)) & 7)); }

template <int TM>
struct MxStageLds {                // one stage of the ring: one LDS object per stage
  uint4 a[MxShape<TM>::kSlotsA];
  uint4 b[MxShape<TM>::kSlotsB];
  uint32_t saw[kBN];               // A scale words of the stage [block row]
  uint32_t sbw[TM];                // B scale words of the stage [token slot]
};

// Per-thread copy sources, fixed for the whole K loop (byte offsets from the
// block-uniform bases): A copy i of a stage moves chunk kDmaA wave + i (rows
// 16 c .. 16 c + 15), the lane taking piece qa[i] of row a[i]; B copy i
// moves chunk kDmaB wave + i (tokens 8 c .. 8 c + 7), the lane taking piece
// pb[i] of the token row at b[i].  Scale words: waves 0-3 copy the words of
// block rows 64 w .. 64 w + 63 (the lane's weight row: sa), the other waves
// those of 64 tokens each (the lane's scale row: sb), several waves copying
// the same bytes to the same slots.  wsm / xsm: stage 0 of the stage-major
// scale words (the block's expert), wrows / xrows: rows per stage.
template <int TM>
struct MxRows {
  const uint8_t* abase;
  const uint8_t* bbase;
  const uint32_t* wsm;
  const uint32_t* xsm;
  uint32_t a[MxShape<TM>::kDmaA], b[MxShape<TM>::kDmaB];
  uint32_t qa[MxShape<TM>::kDmaA], pb[MxShape<TM>::kDmaB];
  uint32_t sa, sb;
  uint32_t wrows, xrows;
  int stages;
};

typedef __attribute__((address_space(3))) void mx_lds_void;
typedef __attribute__((address_space(1))) const void mx_gbl_void;

// 16 (or 4) bytes per lane into the LDS chunk at `dst` (wave-uniform; lane
// L's bytes land at dst + 16 L, or dst + 4 L)
__device__ __forceinline__ void dma16_to_lds(const uint8_t* src, void* dst) {
  __builtin_amdgcn_global_load_lds((mx_gbl_void*)src, (mx_lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const uint8_t* src, void* dst) {
  __builtin_amdgcn_global_load_lds((mx_gbl_void*)src, (mx_lds_void*)dst, 4, 0, 0);
}

// Stage s's copies into LDS: exactly kDmaPerStage copy instructions per
// wave.  Pieces past K are clamped in bounds: their weight operands are
// zeroed at the MFMA (the activation bytes there are copies of real ones, so
// every such product is an exact zero).
template <int TM>
__device__ __forceinline__ void mx_stage_dma(MxStageLds<TM>& d, const MxRows<TM>& rows, int K, int s, int wave) {
  using S = MxShape<TM>;
  const int kblocks = K >> 5;
  const int kb0 = 4 * s;
#pragma unroll
  for (int i = 0; i < S::kDmaA; ++i) {
    const int kb = min(kb0 + (int)rows.qa[i], kblocks - 1);
    dma16_to_lds(rows.abase + rows.a[i] + (uint32_t)kb * 16u, d.a + 64 * (S::kDmaA * wave + i));
  }
#pragma unroll
  for (int i = 0; i < S::kDmaB; ++i) {
    const int kp = min(kBK * s + 16 * (int)rows.pb[i], K - 16);
    dma16_to_lds(rows.bbase + rows.b[i] + (uint32_t)kp, d.b + 64 * (S::kDmaB * wave + i));
  }
  // scale words: waves 0-3 one chunk of 64 weight rows each, the others one
  // chunk of 64 tokens (chunk (wave + 4) % (TM / 64))
  const uint32_t sc = (uint32_t)min(s, rows.stages - 1);
  const uint8_t* wsrc = reinterpret_cast<const uint8_t*>(rows.wsm + sc * rows.wrows + rows.sa);
  const uint8_t* xsrc = reinterpret_cast<const uint8_t*>(rows.xsm + sc * rows.xrows + rows.sb);
  const bool rows_chunk = wave < 4;                    // wave-uniform
  dma4_to_lds(rows_chunk ? wsrc : xsrc,
              rows_chunk ? d.saw + 64 * wave : d.sbw + 64 * ((wave + 4) % (TM / 64)));
}

// Tile t of the gx x gy block tiles (gx over weight rows, gy over tokens):
// tiles are dealt to the 8 XCDs in contiguous chunks (block b runs on XCD
// b % 8), and inside a chunk 32 consecutive tiles form a 4 x 8 patch of
// (row tiles x token tiles), so the blocks one XCD runs at a time share
// their weight and activation tiles in that XCD's L2.
__device__ __forceinline__ bool mx_tile_of_block(int b, int gx, int gy, int* x, int* y) {
  const int T = gx * gy;
  const int per = (T + 7) / 8;
  const int t = (b & 7) * per + (b >> 3);
  if (t >= T) return false;
  constexpr int GX = 4;
  const int g = t / (GX * gy);                // group of GX row tiles
  const int gw = min(GX, gx - g * GX);        // its width (the last group may be narrower)
  const int r = t - g * GX * gy;
  *x = g * GX + r % gw;
  *y = r / gw;
  return true;
}

enum MxMode { kMxDense = 0, kMxGateUp = 1, kMxDown = 2 };

struct MxArgs {
  const uint8_t* wc;                // weight codes (expert 0 in the grouped modes)
  int64_t stride_c;                 // bytes between experts
  const uint32_t* wsm;              // weight scale words, stage-major [E][stages][N]
  const uint8_t* xc;                // activation codes [rows][K]
  const uint32_t* xsm;              // activation scale words [stages][xrows]
  int64_t xrows;                    // rows of xsm per stage: dense M, grouped: the grouped rows
  int64_t N;                        // weight rows (dense, down); gate_up: 2 I
  int64_t M;                        // dense: tokens
  int K;
  int gx, gy;                       // row tiles; token tiles (grouped: an upper bound)
  // grouped modes: experts' rows in grouped order
  int E;
  int I;                            // gate_up: intermediate size
  const int32_t* row_off;           // [E + 1] first grouped row of each expert
  const int32_t* tile_off;          // [E + 1] first token tile of each expert
  const int32_t* row_src;           // gate_up: activation row of each grouped row
  float* y;                         // dense [M][N]; down [grouped rows][N]
  uint8_t* hc;                      // gate_up: h codes [grouped rows][I]
  uint8_t* hs;                      // gate_up: h scale words, stage-major [I / 128][xrows], as bytes
};

// Block tile of the 256 x TM (weight rows x tokens) product (MxShape): wave
// (row group rg, token group) takes 64 weight rows (two 32-row MFMA tiles)
// and 32 tokens (one 32-token tile): 2 MFMAs per 64-deep step, operands
// read from LDS.  The copies of the next two K stages are in flight while
// the MFMAs run (a ring of three LDS stages).  Four waves per SIMD, from one
// or two blocks, cover each other's LDS reads and barrier waits.
//   kMxDense : y[m][n] = sum_k W[n][k] xq[m][k].
//   kMxGateUp: block (token tile of expert e, 128 intermediate rows): A rows
//              0..127 are gate rows i, 128..255 the up rows I + i, and each
//              wave holds the gate and up sums of the same 32 rows, so
//              h = silu(g) * u is formed in registers and quantized to MXFP8
//              along the intermediate axis (a 32-row MFMA tile is one block)
//              straight into the down product's operand.
//   kMxDown  : d[r][n] = sum_i Wd_e[n][i] hq[r][i] for the expert's grouped rows r.
template <int MODE, int TM>
__global__ void __launch_bounds__(MxShape<TM>::kThreads, 4) mx_gemm_kernel(MxArgs p) {
  using S = MxShape<TM>;
  // three separate LDS objects, so that the compiler's wait tracking for
  // the copies tells them apart: an access to one ring stage waits only for
  // the copies into that stage
  __shared__ MxStageLds<TM> R0, R1, R2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int K = p.K;
  const int kblocks = K >> 5;

  // the block's tile: weight rows from n0 (or intermediate rows from i0),
  // token slots [0, 128) -> tokens m0 + slot, or grouped rows r0 + slot (< r_end)
  int64_t n0 = 0, m0 = 0;
  int e = 0, r0 = 0, r_end = 0;
  const uint8_t* wc = p.wc;
  const int stages_k = (kblocks + 3) / 4;
  const uint32_t* wsm = p.wsm;
  if (MODE == kMxDense) {
    int tx, ty;
    if (!mx_tile_of_block(blockIdx.x, p.gx, p.gy, &tx, &ty)) return;   // block-uniform
    n0 = (int64_t)tx * kBN;
    m0 = (int64_t)ty * TM;
  } else {
    // gy = the launch's upper bound on token tiles; the XCD-grouped order
    // keeps the token tiles of one expert and row tile on one XCD's L2
    int tx, T;
    if (!mx_tile_of_block(blockIdx.x, p.gx, p.gy, &tx, &T)) return;    // block-uniform
    if (T >= p.tile_off[p.E]) return;                                  // block-uniform
    int lo = 0, hi = p.E;                                              // tile_off[lo] <= T < tile_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.tile_off[mid] <= T) lo = mid; else hi = mid;
    }
    e = lo;
    r0 = p.row_off[e] + (T - p.tile_off[e]) * TM;
    r_end = p.row_off[e + 1];
    wc += (int64_t)e * p.stride_c;
    wsm += (int64_t)e * stages_k * p.N;
    n0 = (int64_t)tx * (MODE == kMxGateUp ? kBN / 2 : kBN);
  }

  // operand rows of the block: A block row br (0..255) -> weight row;
  // token slot t (0..63) -> activation row (b_row), and the row of its scale
  // words (b_srow: the grouped row in the grouped modes, whose scale words
  // are gathered into grouped order beforehand)
  auto a_row = [&](int br) -> int64_t {
    if (MODE == kMxGateUp) {
      int64_t ir = n0 + (br & 127);
      ir = ir < p.I ? ir : p.I - 1;
      return br < 128 ? ir : p.I + ir;
    }
    const int64_t row = n0 + br;
    return row < p.N ? row : p.N - 1;
  };
  auto b_row = [&](int t) -> int64_t {
    if (MODE == kMxDense) {
      const int64_t src = m0 + t;
      return src < p.M ? src : p.M - 1;
    }
    int gr = r0 + t;
    gr = gr < r_end ? gr : r_end - 1;
    return MODE == kMxGateUp ? p.row_src[gr] : gr;
  };
  auto b_srow = [&](int t) -> int64_t {
    if (MODE == kMxDense) return b_row(t);
    const int gr = r0 + t;
    return gr < r_end ? gr : r_end - 1;
  };
  MxRows<TM> rows;
  rows.abase = wc;
  rows.bbase = p.xc;
  rows.wsm = wsm;
  rows.xsm = p.xsm;
  rows.wrows = (uint32_t)p.N;
  rows.xrows = (uint32_t)p.xrows;
  rows.stages = stages_k;
#pragma unroll
  for (int i = 0; i < S::kDmaA; ++i) {
    const int r = 16 * (S::kDmaA * wave + i) + (lane >> 2);  // slot 64 c + lane = 4 r + (lane & 3)
    rows.a[i] = (uint32_t)(a_row(r) * (K >> 1));
    rows.qa[i] = (uint32_t)((lane & 3) ^ (((r >> 1) ^ (r >> 3)) & 3));
  }
#pragma unroll
  for (int i = 0; i < S::kDmaB; ++i) {
    const int t = 8 * (S::kDmaB * wave + i) + (lane >> 3);   // slot 64 c + lane = 8 t + (lane & 7)
    rows.b[i] = (uint32_t)(b_row(t) * K);
    rows.pb[i] = (uint32_t)((lane & 7) ^ ((t ^ (t >> 3)) & 7));
  }
  rows.sa = (uint32_t)a_row(64 * (wave & 3) + lane);
  rows.sb = (uint32_t)b_srow(64 * ((wave + 4) % (TM / 64)) + lane);

  // the wave's A tiles: block rows arow(a) + j; gate_up pairs tile a (gate)
  // with tile a + 2 (up) over the same intermediate rows
  // wave = (row group rg, token group): kTA tiles of 32 rows, 32 tokens;
  // gate_up: tiles a < kTA / 2 are gate rows, a + kTA / 2 the matching up rows
  const int rg = wave % kRowGroups;
  const int wt = (wave / kRowGroups) * 32 * kNB;   // the wave's first token slot
  auto arow = [&](int a) {
    return MODE == kMxGateUp ? (a >= kTA / 2 ? 128 : 0) + rg * 16 * kTA + 32 * (a % (kTA / 2))
                             : rg * 32 * kTA + 32 * a;
  };
  // byte q of a scale word
  auto word_byte = [](uint32_t w, int q) -> int { return (int)((w >> (8 * q)) & 0xFFu); };

  v16f acc[kTA][kNB];
#pragma unroll
  for (int a = 0; a < kTA; ++a)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // stage s's MFMAs from LDS stage d.  TAIL: a last stage with kval < 4 of
  // its 32-blocks inside K; the weights of the others are masked to zero
  // (bitwise, so that no select turns into a branch around the LDS read).
  auto compute = [&](const MxStageLds<TM>& d, int s, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;   // std::bool_constant
    const int kval = kblocks - 4 * s;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (TAIL && ks == 1 && kval <= 2) break;         // block-uniform
      v8i A[kTA], B[kNB];
      int sa[kTA], sb[kNB];
      const int pa = 2 * ks + h;
      const uint32_t keep = TAIL ? 0u - (uint32_t)(pa < kval) : ~0u;
#pragma unroll
      for (int a = 0; a < kTA; ++a) {
        const int r = arow(a) + j;
        const uint4 q = d.a[a_slot(r, pa)];
        A[a][0] = (int)(q.x & keep);
        A[a][1] = (int)(q.y & keep);
        A[a][2] = (int)(q.z & keep);
        A[a][3] = (int)(q.w & keep);
        A[a][4] = A[a][5] = A[a][6] = A[a][7] = 0;
        sa[a] = word_byte(d.saw[r], pa);
        if (TAIL && pa >= kval) sa[a] = 127;            // past K: any finite scale (the byte is padding)
      }
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        const int t = wt + 32 * b + j;
        const uint4 lo = d.b[b_slot(t, 4 * ks + h)];
        const uint4 hi = d.b[b_slot(t, 4 * ks + 2 + h)];
        B[b][0] = (int)lo.x;
        B[b][1] = (int)lo.y;
        B[b][2] = (int)lo.z;
        B[b][3] = (int)lo.w;
        B[b][4] = (int)hi.x;
        B[b][5] = (int)hi.y;
        B[b][6] = (int)hi.z;
        B[b][7] = (int)hi.w;
        sb[b] = word_byte(d.sbw[t], 2 * ks + h);
        if (TAIL && 2 * ks + h >= kval) sb[b] = 127;
      }
#pragma unroll
      for (int a = 0; a < kTA; ++a)
#pragma unroll
        for (int b = 0; b < kNB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[a], B[b], acc[a][b], 4, 0, 0, sa[a], 0,
                                                                       sb[b]);
    }
  };

  // The ring: stage s lives in LDS stage s % 3.  Step s issues stage s + 2's
  // copies, runs stage s's MFMAs, waits until all of this wave's copies but
  // the last kDmaPerStage (stage s + 2's) have landed - the loop issues no
  // other global loads, and copies complete in issue order, so stage s + 1
  // has - and meets the block at an LDS-only barrier, which publishes every
  // wave's stage s + 1.  Stage s + 2's copies stay in flight through the
  // next step's MFMAs.  The loop runs the full stages; a last, partial
  // stage is computed after it.  Stages past K are loaded clamped and never
  // used; the exit waits for all copies.
  constexpr int kDmaPerStage = S::kDmaPerStage;
  constexpr int kWaitLastStage = 0x0F70 | (kDmaPerStage & 15) | ((kDmaPerStage >> 4) << 14);   // gfx9 vmcnt(n)
  static_assert(kDmaPerStage < 64, "vmcnt holds 6 bits");
  const int full = kblocks / 4;
  auto issue = [&](MxStageLds<TM>& d, int s) {
    __builtin_amdgcn_sched_barrier(0);
    mx_stage_dma<TM>(d, rows, K, s, wave);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_for_all_but_last_stage = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLastStage);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto step = [&](int s, const MxStageLds<TM>& cur, MxStageLds<TM>& load) {
    issue(load, s + 2);
    compute(cur, s, std::false_type{});
    wait_for_all_but_last_stage();
    block_sync_lds();
  };
  issue(R0, 0);
  issue(R1, 1);
  wait_for_all_but_last_stage();
  block_sync_lds();
  // one exit from the loop: every path into its head then has the same
  // copies in flight (those of stage s + 1), so the compiler adds no wait
  int s0 = 0;
  for (; s0 + 3 <= full; s0 += 3) {
    step(s0 + 0, R0, R2);
    step(s0 + 1, R1, R0);
    step(s0 + 2, R2, R1);
  }
  if (s0 < full) step(s0, R0, R2);
  if (s0 + 1 < full) step(s0 + 1, R1, R0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // gfx9 encoding: vmcnt(0)
  if (4 * full < kblocks) {               // block-uniform: the partial last stage, published by the last barrier
    const int r = full % 3;
    compute(r == 0 ? R0 : (r == 1 ? R1 : R2), full, std::true_type{});
  }

  if (MODE == kMxGateUp) {
    // h = silu(g) * u; then MXFP8 per (grouped row, 32 intermediate rows):
    // lane (j, h) holds 16 of a tile's 32 rows, lane (j, 1 - h) the rest
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const int gr = r0 + wt + 32 * b + j;
      const bool row_ok = gr < r_end;
#pragma unroll
      for (int a = 0; a < kTA / 2; ++a) {
        const int64_t i0 = n0 + rg * 16 * kTA + 32 * a;      // first intermediate row of the tile
        float hv[16];
        uint32_t amax = 0, bad = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float g = acc[a][b][r], u = acc[a + kTA / 2][b][r];
          hv[r] = g / (1.0f + expf(-g)) * u;
          const uint32_t ab = __float_as_uint(hv[r]) & 0x7FFFFFFFu;
          bad |= ab >= 0x7F800000u ? 1u : 0u;
          amax = max(amax, ab);
        }
        amax = max(amax, (uint32_t)__shfl_xor((int)amax, 32));
        bad |= (uint32_t)__shfl_xor((int)bad, 32);
        const int eb = (int)(amax >> 23);
        int X = amax == 0 ? -127 : eb - 127 - 8;
        X = X < -127 ? -127 : X;
        const float inv = __uint_as_float((uint32_t)(127 - X) << 23);
        if (row_ok && i0 < p.I) {
          uint8_t* hrow = p.hc + (int64_t)gr * p.I;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            uint32_t word = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              word |= (bad ? 0x7Fu : f32_to_e4m3(hv[4 * g4 + q] * inv)) << (8 * q);
            *reinterpret_cast<uint32_t*>(hrow + i0 + 8 * g4 + 4 * h) = word;
          }
          if (h == 0)   // byte (i0 / 32) % 4 of word [i0 / 128][gr]
            p.hs[((i0 >> 7) * p.xrows + gr) * 4 + ((i0 >> 5) & 3)] = (uint8_t)(bad ? 255 : X + 127);
        }
      }
    }
    return;
  }

#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    int64_t orow;                                   // output row: token, or grouped row
    if (MODE == kMxDense) {
      orow = m0 + wt + 32 * b + j;
      if (orow >= p.M) continue;
    } else {
      orow = r0 + wt + 32 * b + j;
      if (orow >= r_end) continue;
    }
    float* yrow = p.y + orow * p.N;
#pragma unroll
    for (int a = 0; a < kTA; ++a) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t row = n0 + arow(a) + 8 * g + 4 * h;
        const float4 v = make_float4(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                                     acc[a][b][4 * g + 3]);
        if (row + 3 < p.N && (p.N & 3) == 0) {
          *reinterpret_cast<float4*>(yrow + row) = v;
        } else {
          if (row + 0 < p.N) yrow[row + 0] = v.x;
          if (row + 1 < p.N) yrow[row + 1] = v.y;
          if (row + 2 < p.N) yrow[row + 2] = v.z;
          if (row + 3 < p.N) yrow[row + 3] = v.w;
        }
      }
    }
  }
}

// Stage-major scale words: dst[e][s][r] = the E8M0 bytes of K blocks
// 4 s .. 4 s + 3 of source row src_row(r) of expert e, byte q = block 4 s + q
// (blocks past K read 127); src_row(r) = gather[r] if given, else r.  A
// block transposes 16 rows x 32 stages through LDS: it reads each row's 128
// scale bytes with consecutive lanes on consecutive bytes, then writes the
// words with consecutive lanes on consecutive rows.  gridDim = (row blocks
// of 16, stage blocks of 32, experts).
constexpr int kStageThreads = 256;
constexpr int kStageRows = 16;
constexpr int kStageChunk = 32;                       // stages per block: 128 scale bytes per row
constexpr int kStagePitch = 4 * kStageChunk + 4;      // LDS bytes per row (a word of padding)

__global__ void __launch_bounds__(kStageThreads)
mx_stage_scales_kernel(const uint8_t* __restrict__ src, int64_t src_stride_e, int kblocks, int64_t rows,
                       const int32_t* __restrict__ gather, int stages, uint32_t* __restrict__ dst) {
  __shared__ __align__(16) uint8_t tile[kStageRows * kStagePitch];
  const int64_t r0 = (int64_t)blockIdx.x * kStageRows;
  const int s0 = blockIdx.y * kStageChunk, e = blockIdx.z;
  const uint8_t* base = src + (int64_t)e * src_stride_e;
  for (int i = threadIdx.x; i < kStageRows * 4 * kStageChunk; i += kStageThreads) {
    const int r = i / (4 * kStageChunk), c = i % (4 * kStageChunk);
    const int64_t row = r0 + r;
    const int kb = 4 * s0 + c;
    uint32_t v = 127u;
    if (row < rows && kb < kblocks) {
      const int64_t sr = gather ? (int64_t)gather[row] : row;
      v = base[sr * kblocks + kb];
    }
    tile[r * kStagePitch + c] = (uint8_t)v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kStageChunk * kStageRows; i += kStageThreads) {
    const int sl = i / kStageRows, r = i % kStageRows;
    const int s = s0 + sl;
    const int64_t row = r0 + r;
    if (s < stages && row < rows)
      dst[((int64_t)e * stages + s) * rows + row] =
          *reinterpret_cast<const uint32_t*>(tile + r * kStagePitch + 4 * sl);
  }
}

static int64_t a256(int64_t x) { return (x + 255) & ~(int64_t)255; }
static int64_t mx_stages(int64_t k) { return (k / 32 + 3) / 4; }

// the stage-major copy of E experts' [rows][k / 32] scale bytes (gather: the
// source row of each of the `rows` output rows, all < the source's rows)
static int launch_stage_scales(const uint8_t* src, int64_t src_stride_e, int64_t k, int64_t rows,
                               const int32_t* gather, int E, uint32_t* dst, hipStream_t s) {
  const int64_t S = mx_stages(k);
  const int64_t bx = (rows + kStageRows - 1) / kStageRows;
  const int64_t by = (S + kStageChunk - 1) / kStageChunk;
  if (bx > 2147483647LL || by > 65535 || E > 65535) return BDG_E_UNSUPPORTED;
  hipLaunchKernelGGL(mx_stage_scales_kernel, dim3((unsigned)bx, (unsigned)by, (unsigned)E), dim3(kStageThreads), 0,
                     s, src, src_stride_e, (int)(k / 32), rows, gather, (int)S, dst);
  return launch_status();
}

// Picks (t, j) of the M x K routing, grouped by expert: row_off / tile_off
// (token tiles of tm rows) per expert, row_src[r] = token of grouped row r,
// pick_row[t K + j] = its grouped row.  One block; counts are exact, the
// order of one expert's rows depends on atomic timing, which changes no
// result (every grouped row is computed on its own and the combine reads
// each pick's row in slot order).  Up to kGroupLdsPicks picks, each thread
// issues all its index loads at once (a loop that loads, then waits on an
// LDS atomic of the loaded value, pays a round trip per pick), the experts
// stay in LDS for the second pass, and row_src is assembled in LDS and then
// written in order (not scattered from one CU).
constexpr int kGroupThreads = 1024;
constexpr int kGroupLdsPicks = 16384;
constexpr int kGroupPer = kGroupLdsPicks / kGroupThreads;

__global__ void __launch_bounds__(kGroupThreads)
moe_group_picks_kernel(const int32_t* __restrict__ idx, int P, int K, int E, int tm, int32_t* __restrict__ row_off,
                       int32_t* __restrict__ tile_off, int32_t* __restrict__ row_src,
                       int32_t* __restrict__ pick_row) {
  __shared__ int cnt[BDG_MAX_EXPERTS];
  __shared__ int off[BDG_MAX_EXPERTS];
  __shared__ uint16_t pe[kGroupLdsPicks];   // expert of each pick (E <= BDG_MAX_EXPERTS < 2^16)
  __shared__ int32_t rows[kGroupLdsPicks];  // row_src, assembled
  const int tid = threadIdx.x;
  const bool staged = P <= kGroupLdsPicks;
  for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
  __syncthreads();
  if (staged) {
    int ev[kGroupPer];
#pragma unroll
    for (int i = 0; i < kGroupPer; ++i) {
      const int q = tid + i * kGroupThreads;
      ev[i] = idx[q < P ? q : P - 1];        // in bounds; unused past P
    }
#pragma unroll
    for (int i = 0; i < kGroupPer; ++i) {
      const int q = tid + i * kGroupThreads;
      if (q < P) {
        const int e = ev[i] < 0 ? 0 : (ev[i] >= E ? E - 1 : ev[i]);
        pe[q] = (uint16_t)e;
        atomicAdd(&cnt[e], 1);
      }
    }
  } else {
    for (int q = tid; q < P; q += kGroupThreads) {
      int e = idx[q];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int r = 0, t = 0;
    for (int e = 0; e < E; ++e) {
      row_off[e] = r;
      tile_off[e] = t;
      off[e] = r;
      r += cnt[e];
      t += (cnt[e] + tm - 1) / tm;
    }
    row_off[E] = r;
    tile_off[E] = t;
  }
  __syncthreads();
  if (staged) {
    for (int q = tid; q < P; q += kGroupThreads) {
      const int r = atomicAdd(&off[pe[q]], 1);
      rows[r] = q / K;
      pick_row[q] = r;
    }
    __syncthreads();
    for (int r = tid; r < P; r += kGroupThreads) row_src[r] = rows[r];
  } else {
    for (int q = tid; q < P; q += kGroupThreads) {
      int e = idx[q];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      const int r = atomicAdd(&off[e], 1);
      row_src[r] = q / K;
      pick_row[q] = r;
    }
  }
}

// y[t] = sum_j w[t][j] * d[pick_row[t K + j]], j in order.
__global__ void __launch_bounds__(256)
moe_prefill_combine_kernel(const float* __restrict__ d, const int32_t* __restrict__ pick_row,
                           const float* __restrict__ w, int H, int K, float* __restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (c >= H) return;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int jj = 0; jj < K; ++jj) {
    const float wj = w[t * K + jj];
    const float4 dv = ldg_f4(d + (int64_t)pick_row[t * K + jj] * H + c);
    v.x = __builtin_fmaf(wj, dv.x, v.x);
    v.y = __builtin_fmaf(wj, dv.y, v.y);
    v.z = __builtin_fmaf(wj, dv.z, v.z);
    v.w = __builtin_fmaf(wj, dv.w, v.w);
  }
  *reinterpret_cast<float4*>(y + (int64_t)t * H + c) = v;
}

}  // namespace bdg

using namespace bdg;

extern "C" int mxfp8_quantize(const void* x, int32_t x_dtype, int64_t m, int64_t k, uint8_t* codes,
                              uint8_t* scales, void* stream) {
  if (!x || !codes || !scales || m < 1 || k < 32 || (k % 32) != 0) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 3u) != 0) return BDG_E_ALIGN;
  const int64_t n = m * k;
  const int64_t blocks = (n / 4 + kQuantThreads - 1) / kQuantThreads;
  if (blocks > 2147483647LL) return BDG_E_UNSUPPORTED;
  hipLaunchKernelGGL(mxfp8_quant_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0, as_stream(stream), x,
                     x_dtype == BDG_BF16 ? 1 : 0, n, codes, scales);
  return launch_status();
}

extern "C" int64_t mx_scale_words_bytes(const bdg_qmat* w, int32_t n_experts) {
  if (!w || w->fmt != BDG_FMT_MXFP4 || n_experts < 1 || w->n < 1 || w->k < 32 || (w->k % 32) != 0) return -1;
  return 4 * (int64_t)n_experts * mx_stages(w->k) * w->n;
}

extern "C" int mx_stage_scales(const bdg_qmat* w, int32_t n_experts, void* out, int64_t out_bytes, void* stream) {
  int st = check_qmat(w, n_experts > 1);
  if (st != BDG_OK) return st;
  if (w->fmt != BDG_FMT_MXFP4 || !out || n_experts < 1) return BDG_E_INVALID;
  if (n_experts > 1 && w->expert_stride_scales == 0) return BDG_E_INVALID;
  if (!aligned16(out)) return BDG_E_ALIGN;
  if (out_bytes < mx_scale_words_bytes(w, n_experts)) return BDG_E_INVALID;
  return launch_stage_scales(static_cast<const uint8_t*>(w->scales), w->expert_stride_scales, w->k, w->n, nullptr,
                             n_experts, static_cast<uint32_t*>(out), as_stream(stream));
}

// the scale words of w for the MX products: its staged copy, else a fresh
// one written into `dst`
static int weight_scale_words(const bdg_qmat& w, int n_experts, uint32_t* dst, hipStream_t s,
                              const uint32_t** words) {
  if (w.mx_scale_words) {
    if (!aligned16(w.mx_scale_words)) return BDG_E_ALIGN;
    *words = static_cast<const uint32_t*>(w.mx_scale_words);
    return BDG_OK;
  }
  *words = dst;
  return launch_stage_scales(static_cast<const uint8_t*>(w.scales), w.expert_stride_scales, w.k, w.n, nullptr,
                             n_experts, dst, s);
}

extern "C" int64_t mx_gemm_workspace(int64_t n, int64_t k, int64_t m) {
  if (n < 1 || m < 1 || k < 32 || (k % 32) != 0) return -1;
  const int64_t S = mx_stages(k);
  return a256(4 * S * n) + a256(4 * S * m);
}

extern "C" int mx_gemm(const bdg_qmat* w, const uint8_t* x_codes, const uint8_t* x_scales, int64_t m, float* y,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  int st = check_qmat(w, false);
  if (st != BDG_OK) return st;
  if (w->fmt != BDG_FMT_MXFP4) return BDG_E_INVALID;
  if (!x_codes || !x_scales || !y || !workspace || m < 1) return BDG_E_INVALID;
  if (!aligned16(x_codes) || !aligned16(workspace)) return BDG_E_ALIGN;
  if (workspace_bytes < mx_gemm_workspace(w->n, w->k, m)) return BDG_E_INVALID;
  // operand rows are addressed by 32-bit byte offsets from the base pointers
  if (w->k > (int64_t)1 << 20 || w->n * (w->k / 2) >= ((int64_t)1 << 32) || m * w->k >= ((int64_t)1 << 32))
    return BDG_E_UNSUPPORTED;
  if (w->mx_scale_words && !aligned16(w->mx_scale_words)) return BDG_E_ALIGN;
  // 128-token blocks (one per CU, half the weight bytes per product) when
  // they still give every CU two rounds of blocks, else 64-token blocks
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return BDG_E_HIP;
  const int64_t gx = (w->n + kBN - 1) / kBN;
  const int tm = gx * ((m + 127) / 128) >= 2 * (int64_t)cus ? 128 : 64;
  const int64_t gy = (m + tm - 1) / tm;
  if (gx * gy + 8 > 2147483647LL) return BDG_E_UNSUPPORTED;
  const int64_t blocks = (gx * gy + 7) / 8 * 8;     // whole chunks for the 8 XCDs
  const int64_t S = mx_stages(w->k);
  uint32_t* xsm = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + a256(4 * S * w->n));
  hipStream_t s = as_stream(stream);
  const uint32_t* wsm = nullptr;
  st = weight_scale_words(*w, 1, static_cast<uint32_t*>(workspace), s, &wsm);
  if (st) return st;
  st = launch_stage_scales(x_scales, 0, w->k, m, nullptr, 1, xsm, s);
  if (st) return st;
  MxArgs a{};
  a.wc = static_cast<const uint8_t*>(w->codes);
  a.wsm = wsm;
  a.xc = x_codes;
  a.xsm = xsm;
  a.xrows = m;
  a.N = w->n;
  a.M = m;
  a.K = (int)w->k;
  a.gx = (int)gx;
  a.gy = (int)gy;
  a.y = y;
  if (tm == 128)
    hipLaunchKernelGGL((mx_gemm_kernel<kMxDense, 128>), dim3((unsigned)blocks), dim3(MxShape<128>::kThreads), 0, s,
                       a);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<kMxDense, 64>), dim3((unsigned)blocks), dim3(MxShape<64>::kThreads), 0, s, a);
  return launch_status();
}

// Workspace of moe_prefill_mx: x codes [m][H] and scales [m][H/32],
// row_off / tile_off [E + 1] each, row_src / pick_row [m K] each, h codes
// [m K][I], stage-major scale words of the grouped x [H/128][m K] and of h
// [I/128][m K], of the gate_up weights [E][H/128][2 I] and of the down
// weights [E][I/128][H], down outputs [m K][H] fp32; each region 256-byte
// aligned.
extern "C" int64_t moe_prefill_mx_workspace(int64_t m, int32_t hidden, int32_t inter, int32_t n_experts,
                                            int32_t top_k) {
  if (m < 1 || hidden < 32 || inter < 32 || n_experts < 1 || top_k < 1) return -1;
  const int64_t P = m * top_k;
  const int64_t SH = mx_stages(hidden), SI = mx_stages(inter);
  return a256(m * hidden) + a256(m * (hidden / 32)) + 2 * a256(4 * (int64_t)(n_experts + 1)) + 2 * a256(4 * P) +
         a256(P * inter) + a256(4 * SH * P) + a256(4 * SI * P) + a256(4 * SH * 2 * (int64_t)inter * n_experts) +
         a256(4 * SI * (int64_t)hidden * n_experts) + a256(4 * P * hidden);
}

extern "C" int moe_router_topk(const void* x, int32_t x_dtype, const float* w_r, const float* b_r, int32_t m,
                               int32_t h, int32_t e, int32_t topk, int32_t flags, float norm_eps, int32_t* idx,
                               float* wts, float* logits, void* stream);

extern "C" int moe_prefill_mx(const bdg_layer_desc* layer, int32_t n_experts, int32_t top_k, const void* x,
                              int32_t x_dtype, int64_t m, float* y, int32_t* topk_idx, float* topk_w,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  if (!layer || !x || !y || !topk_idx || !topk_w || !workspace || m < 1) return BDG_E_INVALID;
  if (n_experts < 1 || top_k < 1 || top_k > n_experts) return BDG_E_INVALID;
  if (n_experts > BDG_MAX_EXPERTS || top_k > BDG_MAX_TOPK) return BDG_E_UNSUPPORTED;
  const bdg_qmat& gu = layer->gate_up;
  const bdg_qmat& dn = layer->down;
  int st = check_qmat(&gu, true);
  if (st) return st;
  st = check_qmat(&dn, true);
  if (st) return st;
  if (gu.fmt != BDG_FMT_MXFP4 || dn.fmt != BDG_FMT_MXFP4) return BDG_E_INVALID;
  const int64_t H = gu.k, I = dn.k;
  if (gu.n != 2 * I || dn.n != H) return BDG_E_INVALID;
  if (n_experts > 1 && (gu.expert_stride_codes == 0 || dn.expert_stride_codes == 0)) return BDG_E_INVALID;
  if (x_dtype != BDG_F32 && x_dtype != BDG_BF16) return BDG_E_INVALID;
  if (!aligned16(x) || !aligned16(y) || !aligned16(workspace)) return BDG_E_ALIGN;
  if (H > 16384 || I > 16384) return BDG_E_UNSUPPORTED;
  const int64_t need = moe_prefill_mx_workspace(m, (int32_t)H, (int32_t)I, n_experts, top_k);
  if (workspace_bytes < need) return BDG_E_INVALID;
  const int64_t P = m * top_k;
  // 32-bit row offsets inside one expert and into the activations / h
  if (P > (int64_t)1 << 30 || m * H >= ((int64_t)1 << 32) || P * I >= ((int64_t)1 << 32) ||
      2 * I * (H / 2) >= ((int64_t)1 << 32))
    return BDG_E_UNSUPPORTED;
  char* wp = static_cast<char*>(workspace);
  uint8_t* xq = reinterpret_cast<uint8_t*>(wp);             wp += a256(m * H);
  uint8_t* xqs = reinterpret_cast<uint8_t*>(wp);            wp += a256(m * (H / 32));
  int32_t* row_off = reinterpret_cast<int32_t*>(wp);        wp += a256(4 * (int64_t)(n_experts + 1));
  int32_t* tile_off = reinterpret_cast<int32_t*>(wp);       wp += a256(4 * (int64_t)(n_experts + 1));
  int32_t* row_src = reinterpret_cast<int32_t*>(wp);        wp += a256(4 * P);
  int32_t* pick_row = reinterpret_cast<int32_t*>(wp);       wp += a256(4 * P);
  const int64_t SH = mx_stages(H), SI = mx_stages(I);
  uint8_t* hq = reinterpret_cast<uint8_t*>(wp);             wp += a256(P * I);
  uint32_t* xsm = reinterpret_cast<uint32_t*>(wp);          wp += a256(4 * SH * P);
  uint32_t* hsm = reinterpret_cast<uint32_t*>(wp);          wp += a256(4 * SI * P);
  uint32_t* gusm = reinterpret_cast<uint32_t*>(wp);         wp += a256(4 * SH * 2 * I * n_experts);
  uint32_t* dnsm = reinterpret_cast<uint32_t*>(wp);         wp += a256(4 * SI * H * n_experts);
  float* d = reinterpret_cast<float*>(wp);
  hipStream_t s = as_stream(stream);

  st = moe_router_topk(x, x_dtype, layer->w_router, layer->b_router, (int32_t)m, (int32_t)H, n_experts, top_k, 0,
                       0.f, topk_idx, topk_w, nullptr, stream);
  if (st) return st;
  st = mxfp8_quantize(x, x_dtype, m, H, xq, xqs, stream);
  if (st) return st;
  // token tiles of 128 grouped rows when the experts average 256 or more
  // (half the weight bytes per product), else of 64 (fewer idle rows in
  // each expert's last tile)
  const int tm = P >= 256 * (int64_t)n_experts ? 128 : 64;
  hipLaunchKernelGGL(moe_group_picks_kernel, dim3(1), dim3(kGroupThreads), 0, s, topk_idx, (int)P, top_k,
                     n_experts, tm, row_off, tile_off, row_src, pick_row);
  st = launch_status();
  if (st) return st;
  // stage-major scale words: both weight matrices (unless staged already),
  // and x's in grouped order
  const uint32_t *gu_words = nullptr, *dn_words = nullptr;
  st = weight_scale_words(gu, n_experts, gusm, s, &gu_words);
  if (st) return st;
  st = weight_scale_words(dn, n_experts, dnsm, s, &dn_words);
  if (st) return st;
  st = launch_stage_scales(xqs, 0, H, P, row_src, 1, xsm, s);
  if (st) return st;
  // token tiles: at most one partial tile per expert beyond P / tm
  const int64_t tiles = (P + tm - 1) / tm + n_experts;
  MxArgs a{};
  a.E = n_experts;
  a.row_off = row_off;
  a.tile_off = tile_off;
  a.row_src = row_src;
  // gate_up: 128 intermediate rows per block (their gate and up rows)
  a.wc = static_cast<const uint8_t*>(gu.codes);
  a.wsm = gu_words;
  a.stride_c = gu.expert_stride_codes;
  a.xc = xq;
  a.xsm = xsm;
  a.xrows = P;
  a.N = 2 * I;
  a.K = (int)H;
  a.I = (int)I;
  a.gx = (int)((I + kBN / 2 - 1) / (kBN / 2));
  a.hc = hq;
  a.hs = reinterpret_cast<uint8_t*>(hsm);
  a.gy = (int)tiles;
  if (tiles * a.gx + 8 > 2147483647LL) return BDG_E_UNSUPPORTED;
  const dim3 grid_a((unsigned)((tiles * a.gx + 7) / 8 * 8));
  if (tm == 128)
    hipLaunchKernelGGL((mx_gemm_kernel<kMxGateUp, 128>), grid_a, dim3(MxShape<128>::kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<kMxGateUp, 64>), grid_a, dim3(MxShape<64>::kThreads), 0, s, a);
  st = launch_status();
  if (st) return st;
  // down: 256 output rows per block over the grouped h rows
  MxArgs b{};
  b.E = n_experts;
  b.row_off = row_off;
  b.tile_off = tile_off;
  b.wc = static_cast<const uint8_t*>(dn.codes);
  b.wsm = dn_words;
  b.stride_c = dn.expert_stride_codes;
  b.xc = hq;
  b.xsm = hsm;
  b.xrows = P;
  b.N = H;
  b.K = (int)I;
  b.gx = (int)((H + kBN - 1) / kBN);
  b.y = d;
  b.gy = (int)tiles;
  if (tiles * b.gx + 8 > 2147483647LL) return BDG_E_UNSUPPORTED;
  const dim3 grid_b((unsigned)((tiles * b.gx + 7) / 8 * 8));
  if (tm == 128)
    hipLaunchKernelGGL((mx_gemm_kernel<kMxDown, 128>), grid_b, dim3(MxShape<128>::kThreads), 0, s, b);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<kMxDown, 64>), grid_b, dim3(MxShape<64>::kThreads), 0, s, b);
  st = launch_status();
  if (st) return st;
  hipLaunchKernelGGL(moe_prefill_combine_kernel, dim3((unsigned)((H / 4 + 255) / 256), (unsigned)m), dim3(256), 0, s,
                     d, pick_row, topk_w, (int)H, top_k, y);
  return launch_status();
}
