// Router projection fused with top-k routing and the FP8 quantization of x.
//
// The router gate scores every token against the routed experts (Qwen 3.5
// TPU page, MoE paragraph of the model description), and the page's roadmap
// item asks for the top-k selection to happen where the scores are computed
// instead of moving the logits between units.  Here one workgroup (8 waves)
// takes 32 tokens against all E experts:
//   0. (a separate small launch) each fp32 router weight is split exactly
//      into three bf16 pieces, hi = bf16(w), mid = bf16(w - hi),
//      lo = w - hi - mid (at most 8 significant bits), stored in the MFMA's
//      lane order so that every operand load below is one contiguous 1 KB;
//   1. logits[t, e] = x[t] . Wr[e] on the matrix cores: every product
//      x * piece is exact in fp32 and v_mfma_f32_32x32x16_bf16 only adds, so
//      the logits carry nothing but fp32 accumulation rounding.  The weight
//      rows are the first operand, so lane (token l % 32) ends with 16
//      experts of its token per 32-expert tile.
//   2. The tile's logits go to LDS (and to the logits buffer).  The same
//      tokens' x rows are quantized to FP8 (one scale per row or per 128
//      elements; a wave loads two rows of up to 4096 elements at a time).
//   3. Each wave routes 4 of the tokens, one per 16-lane row
//      (route_token_row), while the code stores drain.
// Used by moe_forward for batches above the decode sizes when it is given
// no logits (large batches spread over T / 32 workgroups), and by
// moe_router_front.
#include "quant_dev.h"
#include "route_dev.h"

#include <utility>

namespace moe {

typedef __bf16 v8bf_r __attribute__((ext_vector_type(8)));
typedef float v16f_r __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_r __attribute__((ext_vector_type(4)));

template <typename F, int... Is>
__device__ __forceinline__ void static_for_r(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_r(f, std::make_integer_sequence<int, N>{});
}

constexpr int kRouterTokens = 32;
constexpr int kRouterMaxE = 512;

struct RouterArgs {
    const uint16_t* x;
    const u32x4_r* prep;       // the prepared router weight (router_prep_kernel)
    int T, D, E, k;
    int n_groups, topk_groups;
    const float* sel_bias;
    int renormalize;
    float route_scale;
    float* logits;             // [T, E]
    int* ids;                  // [T, k]
    float* w;                  // [T, k]
    uint8_t* xq;               // codes [T, D] (FP8) or [T, D/2] (MXFP4); NULL for bf16 layers
    void* xs;                  // fp32 scales [T] or [T, D/128], or E8M0 bytes [T, D/32]
};

// w == hi + mid + lo exactly, each piece a bf16 (see the file comment).
__device__ __forceinline__ void split3(float w, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
    hi = f32_to_bf16(w);
    const float r1 = w - bf16_to_f32(hi);        // exact
    mid = f32_to_bf16(r1);
    lo = f32_to_bf16(r1 - bf16_to_f32(mid));     // exact, and exactly a bf16
}

// Prepared router weight: for 32-expert tile et, K step s (64 elements),
// 16-wide chunk c and piece p (0 hi, 1 mid, 2 lo) one 1 KB block in MFMA
// lane order -- lane l = (r, kh) holds the 8 bf16 pieces of expert
// 32 et + r, elements [64 s + 32 kh + 8 c, +8) -- so that every operand load
// of the router kernel is one contiguous 1 KB (8 whole lines) per wave.
// Block ((et * nsteps + s) * 4 + c) * 3 + p; experts past E are zero.
__host__ __device__ inline int64_t router_prep_bytes(int E, int D) {
    return static_cast<int64_t>((E + 31) / 32) * (D / 64) * 12 * 1024;
}

__global__ void __launch_bounds__(256) router_prep_kernel(const float* __restrict__ wr, int E, int D,
                                                          uint16_t* __restrict__ prep) {
    const int nsteps = D >> 6;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (et, s, c, lane)
    const int64_t n = static_cast<int64_t>((E + 31) / 32) * nsteps * 4 * 64;
    if (i >= n) return;
    const int l = static_cast<int>(i & 63), c = static_cast<int>((i >> 6) & 3);
    const int64_t es = i >> 8;                        // et * nsteps + s
    const int s = static_cast<int>(es % nsteps), et = static_cast<int>(es / nsteps);
    const int e = et * 32 + (l & 31);
    const int k0 = 64 * s + 32 * (l >> 5) + 8 * c;
    uint16_t h[8], m[8], lo[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float w = e < E ? wr[static_cast<int64_t>(e) * D + k0 + q] : 0.0f;
        split3(w, h[q], m[q], lo[q]);
    }
    u32x4_r* out = reinterpret_cast<u32x4_r*>(prep) + ((es * 4 + c) * 3) * 64 + l;
    out[0] = __builtin_bit_cast(u32x4_r, h);
    out[64] = __builtin_bit_cast(u32x4_r, m);
    out[128] = __builtin_bit_cast(u32x4_r, lo);
}

// EPT: 32-expert tiles per wave (E <= 128 * EPT); EPL: experts per lane in
// the top-k (E <= 64 * EPL); GROUP: -1 (bf16 layer, x not quantized), 0 (per
// row), 128 (1x128 groups), 32 (MXFP4).
//
// 8 waves: wave w takes the expert tiles w % 4, w % 4 + 4, ... over one half
// of K (w / 4), so two waves per SIMD keep loads in flight; the second half's
// partial sums are added to the first's through LDS in a fixed order (the
// result does not depend on timing).  Each half's x rows move through LDS
// two K steps (128 elements) at a time: the four waves of the half load the
// 32 rows x 256 bytes with 16 lanes per row (whole lines), the next chunk's
// loads in flight while the current chunk multiplies.  The prepared weight
// pieces go straight to registers, one or two (step, tile) units loading while
// the current one multiplies (a ring at constant indices).
template <int EPT, int EPL, int SCORING, int GROUP>
__global__ void __launch_bounds__(512) router_front_kernel(const RouterArgs p) {
    constexpr int LD = EPT * 128 + 1;                       // logits row stride (floats)
    constexpr int XROW = 2 * 128 + 16;                      // staged x row: 2 steps of 128 bytes + pad
    constexpr int XBUF = kRouterTokens * XROW;              // one half's chunk buffer
    constexpr int X_BYTES = 2 * 2 * XBUF;                   // [half][buffer]
    constexpr int LG_BYTES = kRouterTokens * LD * 4;
    constexpr int PART_BYTES = 4 * EPT * 16 * 64 * 4;
    constexpr int RAW = X_BYTES > LG_BYTES + PART_BYTES ? X_BYTES : LG_BYTES + PART_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t s_raw[RAW];
    // the x staging area is reused after the K loop for the logits and the
    // second half's partial sums
    float (*s_lg)[LD] = reinterpret_cast<float (*)[LD]>(s_raw);
    float (*s_part)[EPT][16][64] = reinterpret_cast<float (*)[EPT][16][64]>(s_raw + LG_BYTES);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tg = wave & 3, half = wave >> 2;
    const int t0 = blockIdx.x * kRouterTokens;
    const int r = lane & 31, kh = lane >> 5;
    const int nsteps = p.D >> 6;
    const int s_beg = half * (nsteps >> 1);
    const int nchunks = nsteps >> 2;                        // 2-step chunks per half (D % 256 == 0)

    // x staging: thread tg * 64 + lane of this half copies 16-byte segment
    // (idx % 16) of row idx / 16, idx = that thread + 256 rho (rho = 0, 1)
    const int cthr = tg * 64 + lane;
    const uint8_t* xsrc[2];
    int xdst[2];
#pragma unroll
    for (int rho = 0; rho < 2; ++rho) {
        const int idx = cthr + 256 * rho, row = idx >> 4, seg = idx & 15;
        const int tok = min(t0 + row, p.T - 1);             // rows past T read the last token (not used)
        xsrc[rho] = reinterpret_cast<const uint8_t*>(p.x) + (static_cast<int64_t>(tok) * p.D + 64 * s_beg) * 2 +
                    seg * 16;
        xdst[rho] = half * 2 * XBUF + row * XROW + seg * 16;
    }
    u32x4_r xg[2];
    auto xload = [&](int ch) {
#pragma unroll
        for (int rho = 0; rho < 2; ++rho) xg[rho] = *reinterpret_cast<const u32x4_r*>(xsrc[rho] + ch * 256);
    };
    auto xstore = [&](int buf) {
#pragma unroll
        for (int rho = 0; rho < 2; ++rho) *reinterpret_cast<u32x4_r*>(s_raw + xdst[rho] + buf * XBUF) = xg[rho];
    };

    // Lane (r, kh) supplies, for K step s and chunk c, the elements
    // [64 s + 32 kh + 8 c, +8) of its token row (from LDS) and of its expert
    // rows (prepared): both operands use the same K positions.
    const u32x4_r* wp[EPT];
    bool tile_on[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        const int et = tg + 4 * j;
        tile_on[j] = et * 32 < p.E;
        wp[j] = p.prep + static_cast<int64_t>(tile_on[j] ? et : 0) * nsteps * 12 * 64 + lane;
    }
    v16f_r acc[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[j] = v16f_r{};

    // weight ring slots: three (two units ahead) with one expert tile per
    // wave, two where more tiles' sums leave too few registers for a third
    constexpr int NSLOT = EPT >= 2 ? 2 : 3;
    u32x4_r xa[2][4], wa[NSLOT][12];
    auto wload = [&](auto B, int s, int j) {
        constexpr int b = decltype(B)::value;
#pragma unroll
        for (int q = 0; q < 12; ++q) wa[b][q] = wp[j][(static_cast<int64_t>(s) * 12 + q) * 64];
    };
    auto compute = [&](auto B, auto DS, int j) {
        constexpr int b = decltype(B)::value, ds = decltype(DS)::value;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const v8bf_r xb = __builtin_bit_cast(v8bf_r, xa[ds][c]);
            // smallest pieces first
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf_r, wa[b][3 * c + 2]), xb, acc[j],
                                                             0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf_r, wa[b][3 * c + 1]), xb, acc[j],
                                                             0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf_r, wa[b][3 * c]), xb, acc[j],
                                                             0, 0, 0);
        }
    };

    // Weight units (K step, expert tile) in order: unit 2 EPT ch + u is step
    // s_beg + 2 ch + u / EPT, tile u % EPT.  The ring keeps NSLOT - 1 units
    // in flight ahead of the one being multiplied (unit U in slot U % NSLOT);
    // chunks are unrolled by UNR so that every slot index is a constant.
    // Inside a chunk every load is unconditional (a unit past the end reloads
    // the last one, unused) so that the compiler's waits count exactly the
    // loads issued after the one awaited; a conditional load would make it
    // wait for all of them.  Each half has at least one chunk.
    constexpr int AHEAD = NSLOT - 1;
    constexpr int UNR = (2 * EPT) % NSLOT == 0 ? 1 : NSLOT;
    const int s_end = s_beg + 2 * nchunks;
    auto chunk = [&](auto CC, int ch) __attribute__((always_inline)) {
        constexpr int cc = decltype(CC)::value;             // ch % UNR
        const int buf = ch & 1, s = s_beg + 2 * ch;
        xload(min(ch + 1, nchunks - 1));                    // in flight during this chunk
        // this chunk's x fragments of both steps
        const uint8_t* xs = s_raw + half * 2 * XBUF + buf * XBUF + r * XROW + kh * 64;
#pragma unroll
        for (int ds = 0; ds < 2; ++ds)
#pragma unroll
            for (int c = 0; c < 4; ++c) xa[ds][c] = *reinterpret_cast<const u32x4_r*>(xs + ds * 128 + c * 16);
        static_for<2 * EPT>([&](auto U) {
            constexpr int u = decltype(U)::value;
            constexpr int ul = 2 * EPT * cc + u;                // unit within the unrolled chunks
            constexpr int j = u % EPT;
            // unit + AHEAD: dch chunks on, position u2 there
            constexpr int dch = (u + AHEAD) / (2 * EPT), u2 = (u + AHEAD) % (2 * EPT);
            using Cur = std::integral_constant<int, ul % NSLOT>;
            using Nxt = std::integral_constant<int, (ul + AHEAD) % NSLOT>;
            using DS = std::integral_constant<int, u / EPT>;
            wload(Nxt{}, min(s + 2 * dch + u2 / EPT, s_end - 1), u2 % EPT);
            if (tile_on[j]) compute(Cur{}, DS{}, j);
        });
        // the last chunk stores its reloaded x into the idle buffer (read by
        // no one; the barrier orders it before the buffers' reuse below)
        xstore(buf ^ 1);
        __syncthreads();
    };
    xload(0);
    xstore(0);
    static_for<AHEAD>([&](auto U) {
        constexpr int u = decltype(U)::value;
        wload(std::integral_constant<int, u>{}, s_beg + u / EPT, u % EPT);
    });
    __syncthreads();
    const int nfull = nchunks - nchunks % UNR;
    for (int ch0 = 0; ch0 < nfull; ch0 += UNR)
        static_for<UNR>([&](auto CC) { chunk(CC, ch0 + decltype(CC)::value); });
    static_for<UNR>([&](auto CC) {
        if (nfull + decltype(CC)::value < nchunks) chunk(CC, nfull + decltype(CC)::value);
    });

    // second half -> LDS; first half adds it (fixed order) and owns the tile
    if (half) {
#pragma unroll
        for (int j = 0; j < EPT; ++j)
            if (tile_on[j])
#pragma unroll
                for (int v = 0; v < 16; ++v) s_part[tg][j][v][lane] = acc[j][v];
    }
    __syncthreads();
    // lane (r, kh): token r, register v holds expert 8 (v / 4) + 4 kh + v % 4 of the tile
    if (!half) {
        const bool tok_ok = t0 + r < p.T;
#pragma unroll
        for (int j = 0; j < EPT; ++j) {
            if (!tile_on[j]) continue;
            const int ebase = (tg + 4 * j) * 32;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = ebase + 8 * g + 4 * kh + i;
                    const float l = acc[j][4 * g + i] + s_part[tg][j][4 * g + i][lane];
                    if (e < p.E) {
                        s_lg[r][e] = l;
                        if (tok_ok) p.logits[static_cast<int64_t>(t0 + r) * p.E + e] = l;
                    }
                }
            }
        }
    }
    __syncthreads();

    // The tail: the 32 tokens' x rows in the layer's activation format, then
    // their top-k.  Wave w quantizes rows w, w + 8, w + 16, w + 24; rows of
    // at most 4096 elements (one scale per row or per 128) are loaded two at
    // a time, so the wave waits for two round trips, not four, and the code
    // stores drain while the routing runs.
    if constexpr (GROUP == 0 || GROUP == 128) {
        if (p.D <= 4096) {
            constexpr int XR = 2;   // rows in flight together (four spill registers)
            const int nvec = p.D >> 3;
#pragma unroll
            for (int q0 = 0; q0 < 4; q0 += XR) {
                bf16x8 xv[XR][8];
#pragma unroll
                for (int q = 0; q < XR; ++q) {
                    const int t = min(t0 + wave + 8 * (q0 + q), p.T - 1);
                    const bf16x8* xr = reinterpret_cast<const bf16x8*>(p.x + static_cast<int64_t>(t) * p.D);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int c = lane + 64 * i;
                        xv[q][i] = c < nvec ? ld_once(xr + c) : bf16x8{};
                    }
                }
#pragma unroll
                for (int q = 0; q < XR; ++q) {
                    const int64_t t = t0 + wave + 8 * (q0 + q);
                    if (t < p.T)
                        quant_row_regs<GROUP>(xv[q], p.D, p.xq + t * p.D,
                                              static_cast<float*>(p.xs) + t * (GROUP == 128 ? p.D / 128 : 1), lane);
                }
            }
        } else {
            for (int tt = wave; tt < kRouterTokens; tt += 8) {
                const int t = t0 + tt;
                if (t >= p.T) break;
                quant_x_row<GROUP>(p.x, p.D, t, p.xq, p.xs, lane);
            }
        }
    } else if constexpr (GROUP >= 0) {
        for (int tt = wave; tt < kRouterTokens; tt += 8) {
            const int t = t0 + tt;
            if (t >= p.T) break;
            quant_x_row<GROUP>(p.x, p.D, t, p.xq, p.xs, lane);
        }
    }

    // top-k from the logits in LDS: four tokens per wave, a 16-lane row
    // each; grouped scoring with more than 16 groups routes one token per
    // wave
    if (SCORING == 0 || p.n_groups <= 16) {
        const int tt = 4 * wave + (lane >> 4), t = t0 + tt, j = lane & 15;
        int id;
        float wt;
        route_token_row<4 * EPL, SCORING>(&s_lg[tt][0], p.E, p.k, p.n_groups, p.topk_groups, p.sel_bias,
                                          p.renormalize, p.route_scale, lane, &id, &wt);
        if (t < p.T && j < p.k) {
            p.ids[static_cast<int64_t>(t) * p.k + j] = id;
            p.w[static_cast<int64_t>(t) * p.k + j] = wt;
        }
    } else {
        for (int tt = wave; tt < kRouterTokens; tt += 8) {
            const int t = t0 + tt;
            if (t >= p.T) break;
            int id;
            float wt;
            route_token<EPL, SCORING>(&s_lg[tt][0], p.E, p.k, p.n_groups, p.topk_groups, p.sel_bias,
                                      p.renormalize, p.route_scale, lane, &id, &wt);
            if (lane < p.k) {
                p.ids[static_cast<int64_t>(t) * p.k + lane] = id;
                p.w[static_cast<int64_t>(t) * p.k + lane] = wt;
            }
        }
    }
}

template <int EPT, int EPL, int SCORING>
static void router_launch_group(int group, dim3 g, hipStream_t s, const RouterArgs& a) {
    if (group < 0) hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, -1>), g, dim3(512), 0, s, a);
    else if (group == 0) hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, 0>), g, dim3(512), 0, s, a);
    else if (group == 32) hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, 32>), g, dim3(512), 0, s, a);
    else hipLaunchKernelGGL((router_front_kernel<EPT, EPL, SCORING, 128>), g, dim3(512), 0, s, a);
}

template <int EPT, int EPL>
static void router_launch_scoring(int scoring, int group, dim3 g, hipStream_t s, const RouterArgs& a) {
    if (scoring == MOE_SCORING_SOFTMAX) router_launch_group<EPT, EPL, 0>(group, g, s, a);
    else router_launch_group<EPT, EPL, 1>(group, g, s, a);
}

bool router_front_ok(int E, int D) { return E <= kRouterMaxE && D % 256 == 0; }

int64_t router_front_scratch_bytes(int E, int D) { return router_prep_bytes(E, D); }

// group: -1 (no x quantization), 0, 128 or 32 (MXFP4).  scratch: at least
// router_front_scratch_bytes(E, D) bytes, 16-byte aligned.  The caller has
// validated the layer (router_front_ok, routing limits).
int32_t router_front_launch(const moe_layer_desc* L, const void* x, int T, int group, float* logits, int* ids,
                            float* w, uint8_t* xq, float* xs, void* scratch, hipStream_t s) {
    if (T == 0) return MOE_OK;
    const int E = L->E, D = L->D;
    const int64_t nthreads = static_cast<int64_t>((E + 31) / 32) * (D / 64) * 4 * 64;
    hipLaunchKernelGGL(router_prep_kernel, dim3(static_cast<unsigned>(ceil_div(nthreads, 256))), dim3(256), 0, s,
                       L->router_w, E, D, static_cast<uint16_t*>(scratch));
    RouterArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.prep = static_cast<const u32x4_r*>(scratch);
    a.T = T;
    a.D = D;
    a.E = E;
    a.k = L->top_k;
    a.n_groups = L->n_groups;
    a.topk_groups = L->topk_groups;
    a.sel_bias = L->sel_bias;
    a.renormalize = L->renormalize;
    a.route_scale = L->route_scale;
    a.logits = logits;
    a.ids = ids;
    a.w = w;
    a.xq = xq;
    a.xs = xs;
    const dim3 g(static_cast<unsigned>(ceil_div(T, kRouterTokens)));
    if (E <= 64) router_launch_scoring<1, 1>(L->scoring, group, g, s, a);
    else if (E <= 128) router_launch_scoring<1, 2>(L->scoring, group, g, s, a);
    else if (E <= 256) router_launch_scoring<2, 4>(L->scoring, group, g, s, a);
    else router_launch_scoring<4, 8>(L->scoring, group, g, s, a);
    return moe_launch_status();
}

}  // namespace moe
