// conv_gemm.hip -- implicit-GEMM convolutions on the gfx950 matrix cores.
//
// One kernel template serves every convolution of the decoder:
//   * Conv1d k=7 at dilation d (conv_in, residual conv1): 7 taps at frame
//     offsets j*d - 3d;
//   * Conv1d k=1 (residual conv2, dec_in_proj, the encoder's projection):
//     1 tap;
//   * Conv1d k=3 (the encoder's conv_out): 3 taps at offsets -1, 0, 1;
//   * the encoder's strided Conv1d k=2s, stride s, pad s/2 (minimaxmusic.cpp
//     ARCHITECTURE, "Flow VAE"): with the phase streams
//     x'_p[m] = x[m*s + p - s/2] the output is
//     y[n] = sum_p (w[p] x'_p[n] + w[s + p] x'_p[n + 1]), i.e. a 2-tap conv
//     over s*C phase channels read with an input row stride of s (TAG 2);
//   * ConvTranspose1d k=2s stride s as a polyphase GEMM: output phase r of
//     input frame q is x[q] w[:, :, r] + x[q-1] w[:, :, s+r], i.e. 2 taps at
//     offsets 0 and -1 with M = s*Cout rows m = r*Cout + o.  The transposed
//     conv is a scatter of kernel copies (the col2im_1d overlap-add of the
//     qwentts.cpp ARCHITECTURE page, "Custom GGML ops"); grouping the
//     scattered outputs by phase turns it into a dense GEMM with no column
//     matrix and no zero-stuffing.
//
// GEMM view: D[m][n] = sum_{tap, i} W[tap][m][i] * X[n + off(tap)][i],
// m = output feature, n = output position, reduction over input channels i
// (and taps).  The matrix-core "A" operand is the packed weight tile, "B" is
// the activation tile.  Per 64-byte channel chunk the workgroup stages
//   X rows [n0 + min_off, n0 + BN + max_off)  (the dilation halo included)
//   W      [TAPS][BM] rows
// into LDS once and every tap reads its shifted window of the same X tile.
// Chunks stream through an NS-stage LDS ring by global -> LDS DMA: chunk
// c + NS - 1 is requested before the matrix work of chunk c, so NS - 1
// chunks of loads are in flight behind the math (one barrier per chunk).
// The epilogue adds the bias and optionally the residual, stores
// the fp32 result and/or the next layer's Snake of it in the operand dtype,
// so every Snake is evaluated once per element.
//
// Matrix-core instructions (16x16 output blocks, wave64):
//   fp32: v_mfma_f32_16x16x4_f32; bf16: v_mfma_f32_16x16x32_bf16.
// Lane l of a wave supplies row/column (l % 16) and the 16-byte slice
// (l / 16) of the 64-byte chunk; for fp32 the four floats of that slice feed
// four successive 16x16x4 steps (reduction index permuted consistently on
// both operands).  Accumulator register v of lane l holds D[4*(l/16)+v][l%16].
#include "internal.h"
#include "device_math.h"
#include "gemm_common.h"

namespace voc {

// TAG 0/1/3 only separates kernel names per layer kind (1: the input layers
// conv_in and dec_in_proj; 3: the encoder's conv_out and projection; 0: the
// residual convs) so that profilers report them apart.  TAG 2 is the
// strided conv: its input rows are read through phase streams (a runtime
// stride; 1 elsewhere).
// TT: an instance for decoders with two-term bf16 operands: the operand it
// writes (s_out) holds both terms, and the residual stream h (res, h_out)
// holds fp32 elements.  Otherwise one term, and h's element type follows the
// operands (fp32, or fp16 with bf16).
template <int OP, int TAPS, int WMB, int WNB, int WAVES_M, int WAVES_N, int TAG, int NS, bool TT>
__global__ __launch_bounds__(256) void conv_gemm_kernel(const ConvArgs a) {
  constexpr int HO = TT ? OP_F32 : OP;
  constexpr int ST = TT ? 2 : 1;  // terms of the written operand
  constexpr int CH = OpT<OP>::CH;
  constexpr int ES = OpT<OP>::ES;
  constexpr int BM = WAVES_M * WMB * 16;
  constexpr int BN = WAVES_N * WNB * 16;
  constexpr int XROWS = (BN + HaloMax<TAPS>::v + 15) / 16 * 16;
  constexpr int WROWS = TAPS * BM;
  constexpr int XB = XROWS / 16, WB = WROWS / 16, TB = XB + WB;  // 1 KB blocks per stage
  constexpr int STAGE = TB * 1024;
  constexpr int LW = TB / 4;  // fewest blocks any wave issues per stage
  static_assert(BM % 16 == 0 && XROWS % 16 == 0, "LDS tiles come in blocks of 16 rows");
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  static_assert(NS == 1 || (NS - 2) * LW <= 63, "loads in flight must fit vmcnt");
  // Two-term instances with the register-staged single buffer stage each
  // input chunk's high-term and low-term X tiles side by side against one
  // weight tile (the input's low terms are chunk planes Cin/2 .. of x).
  // Paired for the ConvTranspose1d (8-11 % faster than the doubled
  // reduction); the 7-tap GEMM's doubled X staging costs a workgroup per CU
  // and it runs 20 % slower paired, so it keeps the doubled reduction
  // (conv_in, tag 1, reads the one-term latent operand).
  constexpr bool kPair = TT && NS == 1 && TAG == 0 && TAPS == 2;
  constexpr int XT = kPair ? 2 * XROWS : XROWS;
  __shared__ __attribute__((aligned(1024))) unsigned char smem[NS == 1 ? (XT + WROWS) * kRowBytes : NS * STAGE];

  const int tid = threadIdx.x;
  const int total = a.n_tiles * a.m_tiles * a.rows;
  const int L = xcd_remap(blockIdx.x, total);
  // Each XCD runs a contiguous range of L.  With m_fast the M-tiles that
  // share an activation tile run side by side on one XCD, so the tile is
  // fetched from HBM once and the rest hit L2 (chosen when all weights fit
  // in L2 as well); otherwise one weight slice streams the activations.
  int n_tile, m_tile, row;
  if (a.m_fast) {
    m_tile = L % a.m_tiles;
    const int rest = L / a.m_tiles;
    n_tile = rest % a.n_tiles;
    row = rest / a.n_tiles;
  } else {
    n_tile = L % a.n_tiles;
    const int rest = L / a.n_tiles;
    m_tile = rest % a.m_tiles;
    row = rest / a.m_tiles;
  }
  const int n0 = n_tile * BN;
  const int m0 = m_tile * BM;
  const int len = a.row_len[row];
  const int Lin = min(len * a.rate_in, a.T_in);
  const int Lout = min(len * a.rate_out, a.T_out);
  // The whole tile lies beyond this row's valid output: nothing to do.
  if (n0 * a.ups - a.crop >= Lout) return;

  const int tfirst = n0 + a.min_off;
  // A strided conv (stride S) reads its input as S phase streams per
  // channel chunk: virtual chunk c is phase c % S of chunk c / S, whose frame
  // m is input row m * S + c % S - S/2.  S = 1 is the plain conv.
  const int S = TAG == 2 ? a.in_stride : 1;  // compile-time 1 for the other convs
  const int ph0 = TAG == 2 ? -(S / 2) : 0;    // phase streams start s/2 rows early
  const int nchunks = a.Cin / CH * S;
  const unsigned char* xrow = static_cast<const unsigned char*>(a.x) +
                              static_cast<int64_t>(row) * a.Cin * a.T_in * ES;
  const int64_t xplane = static_cast<int64_t>(a.T_in) * kChunkBytes;
  const unsigned char* wbase = static_cast<const unsigned char*>(a.w);
  const int64_t wplane = static_cast<int64_t>(TAPS) * a.M * kChunkBytes;

  // The wave index is uniform per wave; readfirstlane lets the compiler keep
  // it (and the DMA's LDS addresses derived from it) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int lr = lane & 15, lg = lane >> 4;

  // Stage one chunk: block b < XB holds X rows 16b.. (frames tfirst + row;
  // frames outside [-lb, Lin) read as zero); block XB + k holds weight rows
  // 16k.. of the [TAPS][BM] tile (rows past M read the next tap's rows or
  // zeros and only feed output rows that the epilogue drops).  Block b is
  // copied by wave b % 4.
  const uint32_t smem_lds = lds_addr(smem);
  // Frames in [-lb, 0) are read from memory (a stream's carried context);
  // the buffer resource then starts lb frames before frame 0.  Offsets are
  // 32-bit unsigned: a row before the plane wraps to a value past its end
  // (read as zero).  The host keeps every plane and the rows a tile reads
  // past it below 2^32 bytes, so no offset wraps into the plane.
  const uint32_t xv0 = static_cast<uint32_t>((tfirst + lr) * S + ph0 + a.lb) * uint32_t(kChunkBytes) +
                       static_cast<uint32_t>(lg * 16);
  const uint32_t wv0 = static_cast<uint32_t>(m0 + lr) * uint32_t(kChunkBytes) + static_cast<uint32_t>(lg * 16);
  auto issue = [&](int c, int stage) {
    const i4 xs = buf_rsrc(xrow + (c / S) * xplane - static_cast<int64_t>(a.lb) * kChunkBytes,
                           static_cast<uint32_t>(Lin + a.lb) * kChunkBytes);
    const uint32_t xv = xv0 + static_cast<uint32_t>(c % S) * uint32_t(kChunkBytes);
    const i4 ws = buf_rsrc(wbase + c * wplane, static_cast<uint32_t>(wplane));
    const uint32_t dst = smem_lds + stage * STAGE;
#pragma unroll
    for (int u = 0; u < (TB + 3) / 4; ++u) {
      const int b = wave + 4 * u;
      if (b < XB) {
        dma16(xs, xv + static_cast<uint32_t>(b * 1024 * S), dst + b * 1024);
      } else if (b < TB) {
        const int k = b - XB, j = (16 * k) / BM;
        dma16(ws, wv0 + (j * a.M + 16 * k - j * BM) * kChunkBytes, dst + b * 1024);
      }
    }
  };

  f4 acc[WMB][WNB];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  // A residual (the k=1 conv of a residual unit) is read into registers
  // before the K loop so its HBM latency overlaps the matrix work.  The
  // loads are unconditional (row and frame clamped into range; clamped
  // values are never stored): conditional loads make the compiler wait for
  // each one at the branch join, which serialises the prefetch.
  typename HQuad<HO>::T rres[WMB][WNB];  // converted in the epilogue
  if constexpr (TAPS == 1) {
    if (a.res) {
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb) {
        const int m = min(m0 + wm * WMB * 16 + mb * 16 + lg * 4, a.M - 4);
        const int o = m % a.Cout;
        const int64_t hbase = (static_cast<int64_t>(row) * a.Cout + (o & ~15)) * a.T_out + (o & 15);
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) {
          const int n = min(n0 + wn * WNB * 16 + nb * 16 + lr, Lout - 1);
          rres[mb][nb] = load_h4_raw<HO>(a.res, hbase + static_cast<int64_t>(n) * kHChunk);
        }
      }
    }
  }

  if constexpr (NS == 1) {
    // Register-staged single buffer: the loads of chunk c+1 are issued into
    // registers before chunk c's matrix work and stored to LDS after it.
    // Fewer LDS bytes per workgroup than the ring (more workgroups per CU),
    // which pays where the matrix work per chunk is short (bf16).
    constexpr int XU = (XROWS * 4 + 255) / 256;
    constexpr int WU = (WROWS * 4 + 255) / 256;
    const int xrows = BN + a.halo;
    uint4 xr[XU], xl[kPair ? XU : 1], wr[WU];
    const int nsteps = kPair ? nchunks / 2 : nchunks;  // chunk steps (low terms paired)
    auto gload = [&](int c) {
      const unsigned char* xc = xrow + (c / S) * xplane;
      const int ph = c % S;
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int idx = tid + u * 256;
        const int r = unit_row(idx), col = unit_col(idx);
        const int t = (tfirst + r) * S + ph0 + ph;  // input row
        uint4 v = make_uint4(0u, 0u, 0u, 0u), vl = v;
        if (r < xrows && t >= -a.lb && t < Lin) {
          v = *reinterpret_cast<const uint4*>(xc + static_cast<int64_t>(t) * kChunkBytes + col * 16);
          if constexpr (kPair)
            vl = *reinterpret_cast<const uint4*>(xc + nsteps * xplane + static_cast<int64_t>(t) * kChunkBytes +
                                                 col * 16);
        }
        xr[u] = v;
        if constexpr (kPair) xl[u] = vl;
      }
      const unsigned char* wc = wbase + c * wplane;
#pragma unroll
      for (int u = 0; u < WU; ++u) {
        const int idx = tid + u * 256;
        const int r = unit_row(idx), col = unit_col(idx);
        const int j = r / BM, mm = r - j * BM;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r < WROWS && m0 + mm < a.M)
          v = *reinterpret_cast<const uint4*>(
              wc + (static_cast<int64_t>(j) * a.M + m0 + mm) * kChunkBytes + col * 16);
        wr[u] = v;
      }
    };
    unsigned char* Xs = smem;
    unsigned char* Ws = smem + XT * kRowBytes;
    gload(0);
    for (int c = 0; c < nsteps; ++c) {
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int idx = tid + u * 256;
        const int r = unit_row(idx);
        if (r < xrows) {
          *reinterpret_cast<uint4*>(Xs + lds_off(r, unit_col(idx))) = xr[u];
          if constexpr (kPair) *reinterpret_cast<uint4*>(Xs + XROWS * kRowBytes + lds_off(r, unit_col(idx))) = xl[u];
        }
      }
#pragma unroll
      for (int u = 0; u < WU; ++u) {
        const int idx = tid + u * 256;
        const int r = unit_row(idx);
        if (r < WROWS) *reinterpret_cast<uint4*>(Ws + lds_off(r, unit_col(idx))) = wr[u];
      }
      __syncthreads();
      if (c + 1 < nsteps) gload(c + 1);
      const unsigned char* wt = Ws + (wm * WMB * 16) * kRowBytes + lane * 16;
      const int xr0 = a.off0 - a.min_off + wn * WNB * 16 + lr;
      mma_steps<OP, WMB, WNB, TAPS, TAPS == 7>(
          acc, TAPS, [&](int j, int mb) { return wt + (j * BM + mb * 16) * kRowBytes; },
          [&](int j, int nb) { return Xs + lds_off(xr0 + j * a.offstep, lg) + nb * 1024; });
      if constexpr (kPair)  // the same weights against the low-term tile
        mma_steps<OP, WMB, WNB, TAPS, TAPS == 7>(
            acc, TAPS, [&](int j, int mb) { return wt + (j * BM + mb * 16) * kRowBytes; },
            [&](int j, int nb) { return Xs + XROWS * kRowBytes + lds_off(xr0 + j * a.offstep, lg) + nb * 1024; });
      __syncthreads();
    }
  } else {
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nchunks) issue(s, s);
  int stage = 0;
  for (int c = 0; c < nchunks; ++c) {
    // Chunk c has landed once at most (NS - 2) newer stages are in flight
    // (fewer near the end: then wait for everything).
    if (c + NS - 1 <= nchunks)
      wait_vm<(NS - 2) * LW>();
    else
      wait_vm<0>();
    lds_barrier();  // every wave's copy of chunk c is in; chunk c-1's reads are done
    if (c + NS - 1 < nchunks) issue(c + NS - 1, stage == 0 ? NS - 1 : stage - 1);
    const unsigned char* Xs = smem + stage * STAGE;
    const unsigned char* Ws = Xs + XROWS * kRowBytes;
    // A rows start on 16-row blocks (lane-linear reads); B rows start at the
    // tap's shifted frame, any row.
    const unsigned char* wt = Ws + (wm * WMB * 16) * kRowBytes + lane * 16;
    const int xr0 = a.off0 - a.min_off + wn * WNB * 16 + lr;
    mma_steps<OP, WMB, WNB, TAPS, TAPS == 7>(
        acc, TAPS, [&](int j, int mb) { return wt + (j * BM + mb * 16) * kRowBytes; },
        [&](int j, int nb) { return Xs + lds_off(xr0 + j * a.offstep, lg) + nb * 1024; });
    stage = stage + 1 == NS ? 0 : stage + 1;
  }
  }

  // Epilogue.
  if constexpr (OP == OP_BF16 && TAPS == 1) {
    // bf16: the two 16-row blocks of a 32-channel chunk are finished
    // together; one lane exchange (lane ^ 16) gives every lane 8 contiguous
    // channels of the Snake operand, so each frame's 64-byte operand row is
    // written as four 16-byte stores (not eight 8-byte half-row pieces).
    // (Measured faster for the 1-tap GEMM, whose epilogue stores dominate;
    // the 2- and 7-tap GEMMs lose occupancy to the extra registers and keep
    // the plain path.)
    static_assert(WMB % 2 == 0, "16-row blocks come in chunk pairs");
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int mp = 0; mp < WMB; mp += 2) {
      const int m = m0 + wm * WMB * 16 + mp * 16 + lg * 4;  // first block's rows
      if (m >= a.M) continue;                               // uniform per wave
      const int ph = m / a.Cout;
      const int o = m - ph * a.Cout;                        // channels o.., o+16..
      f4 bias[2], sal[2], sinv[2], hsc[2], hsh[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bias[q] = *reinterpret_cast<const f4*>(a.bias + o + 16 * q);
        sal[q] = sinv[q] = hsc[q] = hsh[q] = f4{0.f, 0.f, 0.f, 0.f};
        if (a.s_out && a.s_alpha) {  // else zero parameters: Snake(v; 0, 0) = v exactly
          sal[q] = *reinterpret_cast<const f4*>(a.s_alpha + o + 16 * q);
          sinv[q] = *reinterpret_cast<const f4*>(a.s_invden + o + 16 * q);
        }
        if (a.hs_scale) {
          hsc[q] = *reinterpret_cast<const f4*>(a.hs_scale + o + 16 * q);
          hsh[q] = *reinterpret_cast<const f4*>(a.hs_h + o + 16 * q);
        }
      }
      const int oc = o - lg * 4;                            // chunk's first channel
      const int cofs = (lg & 1) * 16 + (lg & 2) * 4;        // this lane's 8 channels
      const int64_t sbase = (static_cast<int64_t>(row) * a.Cout * ST + oc) * a.T_out + cofs;
      const int64_t slo = static_cast<int64_t>(a.Cout) * a.T_out;  // low-term planes (two terms)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const int n = n0 + wn * WNB * 16 + nb * 16 + lr;
        const int tau = n * a.ups + ph - a.crop;
        const bool ok = n < a.N && tau >= 0 && tau < Lout;
        u4v pk, pl;  // packed Snake operand (and its low term): blocks 0 and 1 (2 dwords each)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          f4 v = acc[mp + q][nb] + bias[q];
          const int oq = o + 16 * q;
          const int64_t hidx = (static_cast<int64_t>(row) * a.Cout + (oq & ~15)) * a.T_out + (oq & 15) +
                               static_cast<int64_t>(tau) * kHChunk;
          if (a.res) {
            if constexpr (TAPS == 1)
              v += h4_to_f4<HO>(rres[mp + q][nb]);
            else if (ok)
              v += load_h4<HO>(a.res, hidx);
          }
          if (a.s_out || a.hs_scale) v = round_h4<HO>(v);  // a Snake follows: start from the stored h
          if (a.h_out && ok) {
            f4 hv = v;
            if (a.hs_scale) {
              hv[0] = snake_f32(v[0], hsc[q][0], hsh[q][0]);
              hv[1] = snake_f32(v[1], hsc[q][1], hsh[q][1]);
              hv[2] = snake_f32(v[2], hsc[q][2], hsh[q][2]);
              hv[3] = snake_f32(v[3], hsc[q][3], hsh[q][3]);
            }
            store_h4<HO>(a.h_out, hidx, hv);
          }
          f4 sv;
          sv[0] = snake_f32(v[0], sal[q][0], sinv[q][0]);
          sv[1] = snake_f32(v[1], sal[q][1], sinv[q][1]);
          sv[2] = snake_f32(v[2], sal[q][2], sinv[q][2]);
          sv[3] = snake_f32(v[3], sal[q][3], sinv[q][3]);
          pk[2 * q] = pack_bf16x2(sv[0], sv[1]);
          pk[2 * q + 1] = pack_bf16x2(sv[2], sv[3]);
          if constexpr (TT) {
            const f4 lv = bf16_lo4(sv);
            pl[2 * q] = pack_bf16x2(lv[0], lv[1]);
            pl[2 * q + 1] = pack_bf16x2(lv[2], lv[3]);
          }
        }
        if (a.s_out) {  // uniform: every lane takes part in the exchange
          // Even lg keeps block 0 and takes its partner's block 0; odd lg
          // keeps block 1 and takes its partner's block 1.
          const bool odd = lg & 1;
          auto exchange = [&](const u4v& p) {
            const uint32_t s0 = __shfl_xor(static_cast<int>(odd ? p[0] : p[2]), 16);
            const uint32_t s1 = __shfl_xor(static_cast<int>(odd ? p[1] : p[3]), 16);
            u4v out;
            if (odd) {
              out[0] = s0; out[1] = s1; out[2] = p[2]; out[3] = p[3];
            } else {
              out[0] = p[0]; out[1] = p[1]; out[2] = s0; out[3] = s1;
            }
            return out;
          };
          const u4v out = exchange(pk);
          if (ok)
            *reinterpret_cast<u4v*>(static_cast<uint16_t*>(a.s_out) + sbase + static_cast<int64_t>(tau) * CH) = out;
          if constexpr (TT) {
            const u4v outl = exchange(pl);
            if (ok)
              *reinterpret_cast<u4v*>(static_cast<uint16_t*>(a.s_out) + sbase + slo +
                                      static_cast<int64_t>(tau) * CH) = outl;
          }
        }
      }
    }
  } else {
  #pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const int m = m0 + wm * WMB * 16 + mb * 16 + lg * 4;
      if (m >= a.M) continue;
      const int ph = m / a.Cout;
      const int o = m - ph * a.Cout;
      const f4 bias = *reinterpret_cast<const f4*>(a.bias + o);
      f4 sal = f4{0.f, 0.f, 0.f, 0.f}, sinv = f4{0.f, 0.f, 0.f, 0.f};
      if (a.s_out && a.s_alpha) {  // else zero parameters: Snake(v; 0, 0) = v exactly
        sal = *reinterpret_cast<const f4*>(a.s_alpha + o);
        sinv = *reinterpret_cast<const f4*>(a.s_invden + o);
      }
      f4 hsc = f4{0.f, 0.f, 0.f, 0.f}, hsh = f4{0.f, 0.f, 0.f, 0.f};
      if (a.hs_scale) {
        hsc = *reinterpret_cast<const f4*>(a.hs_scale + o);
        hsh = *reinterpret_cast<const f4*>(a.hs_h + o);
      }
      const int64_t hbase = (static_cast<int64_t>(row) * a.Cout + (o & ~15)) * a.T_out + (o & 15);
      const int64_t sbase = (static_cast<int64_t>(row) * a.Cout * ST + (o / CH) * CH) * a.T_out + (o % CH);
      const int64_t slo = static_cast<int64_t>(a.Cout) * a.T_out;  // low-term planes (two terms)
  #pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const int n = n0 + wn * WNB * 16 + nb * 16 + lr;
        if (n >= a.N) continue;
        const int tau = n * a.ups + ph - a.crop;
        if (tau < 0 || tau >= Lout) continue;
        f4 v = acc[mb][nb] + bias;
        const int64_t hidx = hbase + static_cast<int64_t>(tau) * kHChunk;
        if (a.res) {
          if constexpr (TAPS == 1)
            v += h4_to_f4<HO>(rres[mb][nb]);
          else
            v += load_h4<HO>(a.res, hidx);
        }
        if (a.s_out || a.hs_scale) v = round_h4<HO>(v);  // a Snake follows: start from the stored h
        if (a.h_out) {
          f4 hv = v;
          if (a.hs_scale) {
            hv[0] = snake_f32(v[0], hsc[0], hsh[0]);
            hv[1] = snake_f32(v[1], hsc[1], hsh[1]);
            hv[2] = snake_f32(v[2], hsc[2], hsh[2]);
            hv[3] = snake_f32(v[3], hsc[3], hsh[3]);
          }
          store_h4<HO>(a.h_out, hidx, hv);
        }
        if (a.s_out) {
          f4 sv;
          sv[0] = snake_f32(v[0], sal[0], sinv[0]);
          sv[1] = snake_f32(v[1], sal[1], sinv[1]);
          sv[2] = snake_f32(v[2], sal[2], sinv[2]);
          sv[3] = snake_f32(v[3], sal[3], sinv[3]);
          store_op4<OP>(a.s_out, sbase + static_cast<int64_t>(tau) * CH, sv);
          if constexpr (TT) store_op4<OP>(a.s_out, sbase + slo + static_cast<int64_t>(tau) * CH, bf16_lo4(sv));
        }
      }
    }
  }
}

// Block-tile families: {m-blocks per wave, n-blocks per wave, waves along M, waves along N}.
#ifndef VOC_NARROW16
#define VOC_NARROW16 1, 2, 1, 4
#endif
#ifndef VOC_NARROW32
#define VOC_NARROW32 2, 2, 1, 4
#endif
struct VariantShape { int wmb, wnb, wav_m, wav_n; };
static constexpr VariantShape kVariants[CV_COUNT] = {
    {4, 8, 2, 2},  // CV_128x256
    {4, 4, 1, 4},  // CV_64x256
    {6, 4, 1, 4},  // CV_96x256
    {4, 4, 2, 2},  // CV_128x128
    {4, 2, 1, 4},  // CV_64x128
    {6, 4, 2, 2},  // CV_192x128
    {VOC_NARROW16},  // CV_16x128
    {VOC_NARROW32},  // CV_32x128
};

int conv_variant_bm(int v) { return kVariants[v].wav_m * kVariants[v].wmb * 16; }
int conv_variant_bn(int v) { return kVariants[v].wav_n * kVariants[v].wnb * 16; }
bool conv_variant_ok(int v, int taps) {
  if (v < 0 || v >= CV_COUNT) return false;
  // Narrow-M tiles: the 7-tap convs, and (fp32 only) the 1- and 2-tap ones.
  if (v == CV_16x128 || v == CV_32x128) return taps == 7 || taps == 1 || taps == 2;
  // All taps' weight rows of a chunk live in LDS: keep two workgroups per CU.
  if (taps == 7 || taps == 3) return v == CV_64x256 || v == CV_96x256 || v == CV_64x128;
  return true;
}

// LDS ring depth per tap count: the 7-tap GEMM has long matrix work per
// chunk, the 1- and 2-tap GEMMs need more chunks in flight to hide latency.
// NS = 1 selects the register-staged single buffer.
#ifndef VOC_NS_F32
#define VOC_NS_F32 2, 3, 4  // taps 7, 2, 1
#endif
#ifndef VOC_NS_BF16
#define VOC_NS_BF16 1, 1, 4
#endif
template <int OP, int TAPS> struct Stages {
  static constexpr int f[3] = {VOC_NS_F32}, b[3] = {VOC_NS_BF16};
  static constexpr int v = (OP == OP_F32 ? f : b)[TAPS == 7 ? 0 : TAPS == 1 ? 2 : 1];  // 2 and 3 taps alike
};

template <int OP, int TAPS, int TAG, bool TT = false>
static hipError_t launch_taps(int variant, const ConvArgs& a, hipStream_t s) {
  constexpr int NS = Stages<OP, TAPS>::v;
  const int total = a.n_tiles * a.m_tiles * a.rows;
  const dim3 grid(total), block(256);
  switch (variant) {
#define VOC_CASE(V, A, B, C, D)                                                            \
  case V:                                                                                  \
    hipLaunchKernelGGL((conv_gemm_kernel<OP, TAPS, A, B, C, D, TAG, NS, TT>), grid, block, 0, s, a); \
    break;
    VOC_CASE(CV_64x256, 4, 4, 1, 4)
    VOC_CASE(CV_96x256, 6, 4, 1, 4)
    VOC_CASE(CV_64x128, 4, 2, 1, 4)
#undef VOC_CASE
#define VOC_CASE(V, A, B, C, D)                                                              \
  case V:                                                                                    \
    if constexpr (TAPS == 1 || TAPS == 2) {                                                  \
      hipLaunchKernelGGL((conv_gemm_kernel<OP, TAPS, A, B, C, D, TAG, NS, TT>), grid, block, 0, s, a); \
      break;                                                                                 \
    }                                                                                        \
    return hipErrorInvalidValue;
    VOC_CASE(CV_128x256, 4, 8, 2, 2)
    VOC_CASE(CV_128x128, 4, 4, 2, 2)
    VOC_CASE(CV_192x128, 6, 4, 2, 2)
#undef VOC_CASE
#define VOC_CASE(V, A, B, C, D)                                                              \
  case V:                                                                                    \
    if constexpr (TAPS == 7 || (OP == OP_F32 && (TAPS == 1 || TAPS == 2))) {                 \
      hipLaunchKernelGGL((conv_gemm_kernel<OP, TAPS, A, B, C, D, TAG, NS, TT>), grid, block, 0, s, a); \
      break;                                                                                 \
    }                                                                                        \
    return hipErrorInvalidValue;
#define VOC_CASE_SHAPE(V, ...) VOC_CASE(V, __VA_ARGS__)  // expands the shape macro first
    VOC_CASE_SHAPE(CV_16x128, VOC_NARROW16)
    VOC_CASE_SHAPE(CV_32x128, VOC_NARROW32)
#undef VOC_CASE_SHAPE
#undef VOC_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_op(int taps, int variant, int tag, const ConvArgs& a, hipStream_t s) {
  if (a.two_term) {  // two-term operands, fp32 residual stream: the decoder's convs only
    if constexpr (OP == OP_BF16) {
      if (a.in_stride > 1 || (tag != 0 && tag != 1)) return hipErrorInvalidValue;
      switch (taps) {
        case 7:
          return tag == 1 ? launch_taps<OP, 7, 1, true>(variant, a, s) : launch_taps<OP, 7, 0, true>(variant, a, s);
        case 2: return launch_taps<OP, 2, 0, true>(variant, a, s);
        case 1: return launch_taps<OP, 1, 0, true>(variant, a, s);
        default: return hipErrorInvalidValue;
      }
    }
    return hipErrorInvalidValue;
  }
  switch (taps) {
    case 7:
      return tag == 1 ? launch_taps<OP, 7, 1>(variant, a, s) : launch_taps<OP, 7, 0>(variant, a, s);
    case 2:
      return a.in_stride > 1 ? launch_taps<OP, 2, 2>(variant, a, s) : launch_taps<OP, 2, 0>(variant, a, s);
    case 3: return launch_taps<OP, 3, 3>(variant, a, s);  // only the encoder's conv_out
    case 1:
      return tag == 1   ? launch_taps<OP, 1, 1>(variant, a, s)
             : tag == 3 ? launch_taps<OP, 1, 3>(variant, a, s)
                        : launch_taps<OP, 1, 0>(variant, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv(int op, int taps, int variant, int tag, const ConvArgs& a, hipStream_t s) {
  return op == OP_F32 ? launch_op<OP_F32>(taps, variant, tag, a, s) : launch_op<OP_BF16>(taps, variant, tag, a, s);
}

}  // namespace voc
