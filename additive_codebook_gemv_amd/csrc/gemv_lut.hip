// Batch-1 decode GEMV through per-group lookup tables.
//
// Drop-by-Drop ("Multi-Bitwidth Quantization for LLMs Using Additive
// Codebooks"), section 3.2 and section 5: a weight group is the sum of the
// codewords its k codes select, so its contribution to an output row is
//     sum_{m<k} T_{m,j}[code(i,j,m)],   T_{m,j}[c] = < C_m[c], xrot[8j .. 8j+8) >.
// For batch 1 every row reuses the same 256-entry table per (group, codebook),
// so the product becomes one 2-byte table lookup and half an fp32 add per code
// byte instead of a 16-byte codeword gather and four dot2 steps.
//
// Work split.  A "slot" is one (group tile, codebook) pair: 64 groups of one
// plane.  A workgroup owns a slice of 4 consecutive slots and a block of row
// tiles.  It builds the 4 x 64 tables of its slice with matrix-core products
// (v_mfma_f32_32x32x8_f16: 32 codewords x 8 elements times 8 elements x 32
// groups), stores them as fp16 in LDS, then streams its row tiles: lane l of a
// wave loads the 16 codes of group l for 16 rows for each slot (one coalesced
// 1 KiB tile per slot), looks up the four table entries of every row and adds
// them in fp32.
//
// LDS layout.  Entry (slot s, codeword c, lane l) is the fp16 at byte
//     (s/2)*64K + c*256 + l*4 + 2*(s%2),
// so lane l only ever touches LDS bank l (mod the bank count): the random
// codes never collide, and the address is built from the code byte with one
// v_perm_b32 (code -> byte 1, lane offset -> byte 0, slot pair -> byte 2).
//
// Reduction.  Each lane holds 16 row partials (its group, all slots).  A
// transposing butterfly (permlane32 swap, permlane16 swap, row mirror, half
// row mirror, quad DPP) leaves row (l >> 2) summed over the wave in lane l.
// Each slice adds its row sums into one 64-bit word per row in the workspace
// (a contribution count plus a fixed-point sum, device-scope integer atomics);
// the lane whose atomic add completes the count holds the exact total, scales
// it by s_i, rounds to fp16, writes y and clears the word.  No barrier or
// counter is needed, results are bit-reproducible, and the workspace is zero
// again when the kernel ends.
#include "fwht_device.h"
#include "lut_device.h"

namespace aqd {

constexpr int LUT_MAX_GROUP = AQD_MAX_GROUP;                  // linears per launch

// One linear of a launch.  Several linears that share the input (and k) run
// in one launch: their workgroups follow each other in the grid.
struct LutLinear {
    const uint8_t* packed;
    const uint16_t* codebooks;
    const uint16_t* scales;
    uint16_t* y;
    unsigned long long* acc;  // workspace: [d_out] counted fixed-point row sums, zero between calls
    int64_t d_out, n_rt, plane_bytes;
    int tiles_per_block;
    int wg_begin;             // first workgroup of this linear
};

struct LutArgs {
    LutLinear lin[LUT_MAX_GROUP];
    const uint16_t* x;
    int64_t G, n_gt;
    int k, n_slots, slices, n_lin;
    const uint64_t* signs;       // rotating launch only: NULL or the input sign mask (bit c of word c / 64)
};

// HB > 0: x is the raw fp16 activation and the workgroup applies the block
// Walsh-Hadamard rotation (block HB) to the inputs its tables need, with the
// butterflies and rounding of the standalone rotation (same bits), after the
// optional sign flips of the randomized variant.
//
// The fields the first loads depend on come first, as scalars, so that the
// launch preloads them into SGPRs (kernel-argument preloading; a by-value
// struct cannot be preloaded): a workgroup then issues its table operand and
// code loads without first waiting for an argument load.  packed0, codebooks0,
// plane_bytes0, n_rt0 and tpb0 are those of linear 0, which a single-linear
// launch uses; the other fields stay in the struct.
template <int WAVES, int K, bool MULTI, int HB, int TPW>
__global__ __launch_bounds__(64 * WAVES) void gemv_lut_kernel(const uint8_t* __restrict__ packed0,
                                                              const uint16_t* __restrict__ codebooks0,
                                                              const uint16_t* __restrict__ xin, int64_t plane_bytes0,
                                                              int n_rt0, int G, int slices, int n_slots, int tpb0,
                                                              LutArgs p) {
    constexpr int XS_BYTES = HB > 0 ? LUT_SLOTS * TILE_GROUPS * GROUP * 2 : 0;   // rotated inputs, fp16
    __shared__ __align__(16) uint8_t lds[LUT_BYTES + XS_BYTES + 16];
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds + LUT_BYTES);              // [slot][512]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // this workgroup's linear (uniform); a single-linear launch reads its fields
    // at fixed offsets, without a second dependent argument load
    int l = 0;
    if (MULTI) {
#pragma unroll
        for (int i = 1; i < LUT_MAX_GROUP; ++i)
            if (i < p.n_lin && (int)blockIdx.x >= p.lin[i].wg_begin) l = i;
    }
    const LutLinear L = p.lin[MULTI ? l : 0];
    const uint8_t* const packed = MULTI ? L.packed : packed0;
    const uint16_t* const codebooks = MULTI ? L.codebooks : codebooks0;
    const int64_t plane_bytes = MULTI ? L.plane_bytes : plane_bytes0;
    const int64_t n_rt = MULTI ? L.n_rt : (int64_t)n_rt0;
    const int tiles_per_block = MULTI ? L.tiles_per_block : tpb0;
    const int local = (int)blockIdx.x - (MULTI ? L.wg_begin : 0);
    const int slice = local % slices;
    const int rb = local / slices;
    const int64_t t0 = (int64_t)rb * tiles_per_block;
    const int64_t t1 = t0 + tiles_per_block < n_rt ? t0 + tiles_per_block : n_rt;

    // slot s of this slice: q = slice*4 + s -> group tile q / K, codebook q % K.
    // Every load below is unconditional (inactive slots, padding groups and
    // missing tiles read a valid address and the value is replaced by zero), so
    // the compiler can wait for exactly the loads a step needs.
    __amdgpu_buffer_rsrc_t slot_buf[LUT_SLOTS];
    bool slot_on[LUT_SLOTS];
#pragma unroll
    for (int s = 0; s < LUT_SLOTS; ++s) {
        const int q = slice * LUT_SLOTS + s;
        slot_on[s] = q < n_slots;
        const int qq = slot_on[s] ? q : 0;
        slot_buf[s] = slot_rsrc(packed + (int64_t)(qq % K) * plane_bytes + (int64_t)(qq / K) * n_rt * TILE_BYTES,
                                n_rt * TILE_BYTES);
    }

    // ---- table operands first (loads complete in order)
    constexpr int ITEMS = 32 / WAVES;
    uint2 av[ITEMS][2], bv[ITEMS][2];
    bool bok[ITEMS][2];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
        const int item = wave + u * WAVES;
        const int cb = (item >> 1) & 7, gb = item & 1, pair = item >> 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q = slice * LUT_SLOTS + 2 * pair + h;
            const int qq = q < n_slots ? q : 0;
            const int e0 = 4 * (lane >> 5);
            const int c = cb * 32 + (lane & 31);
            const int64_t g = (int64_t)(qq / K) * TILE_GROUPS + gb * 32 + (lane & 31);
            bok[u][h] = q < n_slots && g < G;
            const int64_t gc = g < G ? g : G - 1;
            av[u][h] = *reinterpret_cast<const uint2*>(codebooks + ((int64_t)(qq % K) * CODEWORDS + c) * GROUP + e0);
            if (HB == 0) bv[u][h] = *reinterpret_cast<const uint2*>(xin + gc * GROUP + e0);
        }
    }
    // raw activation blocks for the rotation: slot s needs inputs 512*tile .. +512 (tile = q / K),
    // i.e. 512 / HB blocks; wave w takes blocks w, w + WAVES, ...
    constexpr int BLK_PER_SLOT = HB > 0 ? TILE_GROUPS * GROUP / HB : 1;
    constexpr int NBLK = LUT_SLOTS * BLK_PER_SLOT;
    constexpr int BPW = (NBLK + WAVES - 1) / WAVES;
    constexpr int E = HB > 0 ? HB / 64 : 1;
    float xv[BPW][E];
    bool xok[BPW];
    if (HB > 0) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int blk = wave + b * WAVES;
            const int sl = (blk < NBLK ? blk : 0) / BLK_PER_SLOT, j = (blk < NBLK ? blk : 0) % BLK_PER_SLOT;
            const int q = slice * LUT_SLOTS + sl;
            const int64_t in0 = (int64_t)((q < n_slots ? q : 0) / K) * (TILE_GROUPS * GROUP) + (int64_t)j * HB;
            xok[b] = blk < NBLK && q < n_slots && in0 < (int64_t)G * GROUP;
#pragma unroll
            for (int e = 0; e < E; ++e) xv[b][e] = h2f(xin[xok[b] ? in0 + e * 64 + lane : lane]);
            if (p.signs) {                                      // randomized rotation: eps = -1 where the bit is set
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if ((p.signs[xok[b] ? in0 / 64 + e : 0] >> lane) & 1ull) xv[b][e] = -xv[b][e];
            }
        }
    }

    // Vector memory requests of a CU are served in issue order, so a wave's table
    // operands would otherwise queue behind the code tiles other waves issued
    // earlier and the build could only start once the whole stream had arrived.
    // Every wave issues its operand loads before any wave issues a code load.
    __builtin_amdgcn_s_barrier();

    // ---- then the first code tile of every wave: half of the workgroup's code
    // stream is in flight while the tables are built.  The second half is
    // requested only after the build (below): requests issued earlier would sit
    // in front of other workgroups' table operands and delay every build.
    uint4 codes[TPW][LUT_SLOTS];
    auto load_tile = [&](int u) {
        const int64_t it = t0 + wave + (int64_t)u * WAVES;
        const uint32_t off = it < t1 ? (uint32_t)(it * TILE_BYTES) + lane * TILE_ROWS : NO_TILE;
#pragma unroll
        for (int s = 0; s < LUT_SLOTS; ++s) codes[u][s] = load_stream(slot_buf[s], slot_on[s] ? off : NO_TILE);
    };
    load_tile(0);
    // scales of the rows this lane may finish (needed only at the end; clamped)
    uint16_t row_scale[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t row = (t0 + wave + (int64_t)u * WAVES) * TILE_ROWS + (lane >> 2);
        row_scale[u] = L.scales[row < L.d_out ? row : L.d_out - 1];
    }
    if (HB > 0) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int blk = wave + b * WAVES;
            if (blk >= NBLK) continue;                          // uniform over the wave
            if constexpr (HB > 0) fwht_block<HB>(xv[b], lane);
#pragma unroll
            for (int e = 0; e < E; ++e) xs[blk * HB + e * 64 + lane] = xok[b] ? f2h(xv[b][e]) : (uint16_t)0;
        }
        __syncthreads();                                        // rotated inputs of every slot are in LDS
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            const int item = wave + u * WAVES;
            const int gb = item & 1, pair = item >> 4;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                bv[u][h] = *reinterpret_cast<const uint2*>(xs + (2 * pair + h) * (TILE_GROUPS * GROUP) +
                                                           (gb * 32 + (lane & 31)) * GROUP + 4 * (lane >> 5));
        }
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (!bok[u][h]) bv[u][h] = make_uint2(0u, 0u);     // zero activation -> zero table entries
        }

#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
        const int item = wave + u * WAVES;
        const int pair = item >> 4, cb = (item >> 1) & 7, gb = item & 1;
        floatx16_t t[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int r = 0; r < 16; ++r) t[h][r] = 0.f;
            t[h] = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(half4_t, av[u][h]),
                                                        __builtin_bit_cast(half4_t, bv[u][h]), t[h], 0, 0, 0);
        }
        const int gl = gb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = cb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const half2_t v = half2_t{(_Float16)t[0][r], (_Float16)t[1][r]};
            *reinterpret_cast<half2_t*>(lds + pair * LUT_PAIR_BYTES + c * 256 + gl * 4) = v;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 1; u < TPW; ++u) load_tile(u);

    uint32_t base[LUT_SLOTS];
#pragma unroll
    for (int s = 0; s < LUT_SLOTS; ++s) base[s] = (uint32_t)(lane * 4 + 2 * (s & 1)) | ((uint32_t)(s >> 1) << 16);
    const half2_t ones = half2_t{(_Float16)1.0f, (_Float16)1.0f};
    const float one = opaque_one();

    // returned accumulator words are examined only after the last tile, so the
    // atomics' round trips overlap the remaining lookups
    unsigned long long old_word[TPW], term[TPW];
    bool mine[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        mine[u] = false;
        old_word[u] = 0ull;
        term[u] = 0ull;
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t it = t0 + wave + (int64_t)u * WAVES;
        if (it >= t1) break;                   // uniform across the wave
        float rows[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float a = 0.f;
#pragma unroll
            for (int pr = 0; pr < LUT_SLOTS / 2; ++pr) {
                const uint4& c0 = codes[u][2 * pr];
                const uint4& c1 = codes[u][2 * pr + 1];
                const uint32_t w0 = (r >> 2) == 0 ? c0.x : (r >> 2) == 1 ? c0.y : (r >> 2) == 2 ? c0.z : c0.w;
                const uint32_t w1 = (r >> 2) == 0 ? c1.x : (r >> 2) == 1 ? c1.y : (r >> 2) == 2 ? c1.z : c1.w;
                const uint32_t a0 = lut_addr(w0, base[2 * pr], r & 3);
                const uint32_t a1 = lut_addr(w1, base[2 * pr + 1], r & 3);
                const _Float16 e0 = *reinterpret_cast<const _Float16*>(lds + a0);
                const _Float16 e1 = *reinterpret_cast<const _Float16*>(lds + a1);
                // the first pair as one mixed-precision fma (fp16 inputs, fp32 sum), the others
                // packed into one v_dot2 each
                a = pr == 0 ? __builtin_fmaf((float)e0, one, (float)e1)
                            : __builtin_amdgcn_fdot2(half2_t{e0, e1}, ones, a, false);
            }
            rows[r] = a;
        }
        const float sum = fold_rows(rows, lane);
        const int64_t row = it * TILE_ROWS + (lane >> 2);
        if ((lane & 3) == 0 && row < L.d_out) {
            mine[u] = true;
            term[u] = fix_term(sum);
            old_word[u] = atomicAdd(L.acc + row, fix_add_word(term[u]));
        }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        if (!mine[u] || !fix_is_last(old_word[u], slices)) continue;
        // this lane added the last contribution of its row: it holds the complete sum
        const int64_t row = (t0 + wave + (int64_t)u * WAVES) * TILE_ROWS + (lane >> 2);
        if (row >= L.d_out) continue;
        L.y[row] = f2h(h2f(row_scale[u]) * (float)fix_total(old_word[u], term[u], slices));
        __hip_atomic_store(L.acc + row, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---- host side ---------------------------------------------------------------

static size_t acc_bytes(int64_t d_out) { return ((size_t)d_out * 8 + 255) / 256 * 256; }

size_t gemv_lut_workspace_bytes(const Geometry& g) { return acc_bytes(g.d_out); }

bool gemv_lut_supported(const Geometry& g, int batch, int k) {
    return batch == 1 && g.n_gt > 0 && g.n_rt > 0 && g.n_rt <= LUT_MAX_ROW_TILES &&
           lut_slices(g.n_gt, k) <= LUT_MAX_SLICES;
}

bool gemv_lut_grouped_supported(int64_t G, int k, const int64_t* d_out, int n) {
    const int64_t n_gt = (G + TILE_GROUPS - 1) / TILE_GROUPS;
    for (int i = 0; i < n; ++i)
        if ((d_out[i] + TILE_ROWS - 1) / TILE_ROWS > LUT_MAX_ROW_TILES) return false;
    return n_gt > 0 && lut_slices(n_gt, k) <= LUT_MAX_SLICES;
}

size_t gemv_lut_grouped_workspace_bytes(const int64_t* d_out, int n) {
    size_t b = 0;
    for (int i = 0; i < n; ++i) b += acc_bytes(d_out[i]);
    return b;
}

template <bool MULTI, int HB, int TPW>
static void launch_k(int k, dim3 gd, dim3 bd, hipStream_t s, const LutArgs& a) {
    switch (k) {
#define AQD_LUT_ARGS a.lin[0].packed, a.lin[0].codebooks, a.x, a.lin[0].plane_bytes, (int)a.lin[0].n_rt, (int)a.G, \
                     a.slices, a.n_slots, a.lin[0].tiles_per_block, a
        case 1: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 1, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 2: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 2, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 3: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 3, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 4: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 4, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 5: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 5, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 6: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 6, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 7: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 7, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        default: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 8, MULTI, HB, TPW>), gd, bd, 0, s, AQD_LUT_ARGS); break;
#undef AQD_LUT_ARGS
    }
}

template <bool MULTI, int HB>
static void launch_tpw(int tpw, int k, dim3 gd, dim3 bd, hipStream_t s, const LutArgs& a) {
    if (tpw == LUT_TILES_PER_WAVE_BIG) launch_k<MULTI, HB, LUT_TILES_PER_WAVE_BIG>(k, gd, bd, s, a);
    else launch_k<MULTI, HB, LUT_TILES_PER_WAVE>(k, gd, bd, s, a);
}

hipError_t launch_gemv_lut_grouped(const LutLinearRef* lins, int n, int k, const uint16_t* x, int64_t d_in,
                                   void* ws, hipStream_t s, int rotate_block, const uint8_t* signs) {
    const int64_t G = d_in / GROUP;
    const int64_t n_gt = (G + TILE_GROUPS - 1) / TILE_GROUPS;
    LutArgs a = {};
    a.x = x;
    a.signs = rotate_block ? reinterpret_cast<const uint64_t*>(signs) : nullptr;
    a.G = G;
    a.n_gt = n_gt;
    a.k = k;
    a.n_slots = (int)((int64_t)k * n_gt);
    a.slices = lut_slices(n_gt, k);
    int64_t n_rt[LUT_MAX_GROUP];
    int tpb[LUT_MAX_GROUP], blocks[LUT_MAX_GROUP];
    int m = 0;                                 // linears with rows
    for (int i = 0; i < n; ++i)
        if (lins[i].d_out > 0) {
            a.lin[m].packed = lins[i].packed;
            a.lin[m].codebooks = lins[i].codebooks;
            a.lin[m].scales = lins[i].scales;
            a.lin[m].y = lins[i].y;
            a.lin[m].d_out = lins[i].d_out;
            a.lin[m].n_rt = (lins[i].d_out + TILE_ROWS - 1) / TILE_ROWS;
            a.lin[m].plane_bytes = a.lin[m].n_rt * n_gt * TILE_BYTES;
            n_rt[m] = a.lin[m].n_rt;
            ++m;
        }
    if (m == 0) return hipSuccess;
    a.n_lin = m;
    // two row tiles per wave, or four when two would need more workgroups than CUs (a second round)
    const bool round4 = m == 1 && rotate_block == 0;   // the plain single-linear GEMV
    int tpw = LUT_TILES_PER_WAVE;
    lut_plan(n_rt, m, a.slices, tpw, tpb, blocks, round4);
    int64_t wgs = 0;
    for (int i = 0; i < m; ++i) wgs += (int64_t)a.slices * blocks[i];
    if (wgs > LUT_CUS) {
        tpw = LUT_TILES_PER_WAVE_BIG;
        lut_plan(n_rt, m, a.slices, tpw, tpb, blocks, round4);
    }
    uint8_t* acc = static_cast<uint8_t*>(ws);
    int wg = 0;
    for (int i = 0; i < m; ++i) {
        a.lin[i].tiles_per_block = tpb[i];
        a.lin[i].wg_begin = wg;
        a.lin[i].acc = reinterpret_cast<unsigned long long*>(acc);
        acc += acc_bytes(a.lin[i].d_out);
        wg += a.slices * blocks[i];
    }
    const dim3 gd((unsigned)wg), bd(64 * LUT_WAVES);
    // one linear: the instantiation that takes every field its first loads need from the preloaded
    // leading arguments
    const bool one = m == 1;
    if (rotate_block == 64) one ? launch_tpw<false, 64>(tpw, k, gd, bd, s, a) : launch_tpw<true, 64>(tpw, k, gd, bd, s, a);
    else if (rotate_block == 128)
        one ? launch_tpw<false, 128>(tpw, k, gd, bd, s, a) : launch_tpw<true, 128>(tpw, k, gd, bd, s, a);
    else if (rotate_block == 256)
        one ? launch_tpw<false, 256>(tpw, k, gd, bd, s, a) : launch_tpw<true, 256>(tpw, k, gd, bd, s, a);
    else one ? launch_tpw<false, 0>(tpw, k, gd, bd, s, a) : launch_tpw<true, 0>(tpw, k, gd, bd, s, a);
    return hipGetLastError();
}

hipError_t launch_gemv_lut(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                           const uint16_t* x, uint16_t* y, const Geometry& g, void* ws, hipStream_t s) {
    const LutLinearRef one = {packed, codebooks, scales, y, g.d_out};
    return launch_gemv_lut_grouped(&one, 1, k, x, g.d_in, ws, s, 0, nullptr);
}

}  // namespace aqd
