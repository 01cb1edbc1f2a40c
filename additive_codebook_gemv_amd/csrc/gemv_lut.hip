// Batch-1 decode GEMV through per-group lookup tables.
//
// Drop-by-Drop ("Multi-Bitwidth Quantization for LLMs Using Additive
// Codebooks"), section 3.2 and section 5: a weight group is the sum of the
// codewords its k codes select, so its contribution to an output row is
//     sum_{m<k} T_{m,j}[code(i,j,m)],   T_{m,j}[c] = < C_m[c], xrot[8j .. 8j+8) >.
// For batch 1 every row reuses the same 256-entry table per (group, codebook),
// so the product becomes one 2-byte table lookup per code byte instead of a
// 16-byte codeword gather and four dot2 steps.
//
// Work split.  A "slot" is one (group tile, codebook) pair: 64 groups of one
// plane.  A workgroup owns a slice of S consecutive slots (S = 1 at k = 1 on
// inputs under 6144, else 2 at k <= 2, 4 from k = 3 except on linears too
// small to give each wave a row tile and, at k = 3, on long inputs whose
// 2-slot plan fits one round of workgroups, which keep 2; more if a row would
// otherwise take more than 255 contributions) and a block of row tiles.  It
// builds the S x 64 tables of its slice with matrix-core products
// (v_mfma_f32_32x32x8_f16: 32 codewords x 8 elements times 8 elements x 32
// groups) and stores them as fp16 in LDS, then
// streams its row tiles: lane l of a wave loads the 16 codes of group l for 16
// rows for each slot (one coalesced 1 KiB tile per slot) and looks up the
// table entry of every row and slot.  A slot's tables cost the same to build
// whatever the number of rows that use them, so at small k a workgroup takes
// fewer slots and more row tiles.
//
// Order of requests.  All waves first request their table operands (a few KB
// that every workgroup reads); each wave requests its first code tile only
// once its own operands have arrived, and the other tiles after the tables are
// built.  Requested earlier, code tiles sit in front of the operands of
// workgroups that are still waiting for them in the memory queues, and every
// table build waits with them.
//
// LDS layout.  Entry (slot s, codeword c, lane l) is the fp16 at byte
//     (s/2)*64K + c*256 + l*4 + 2*(s%2),
// so lane l only ever touches LDS bank l (mod the bank count): the random
// codes never collide, and the address is built from the code byte with one
// v_perm_b32 (code -> byte 1, lane offset -> byte 0, slot pair -> byte 2).
//
// Reduction.  The entries of 4 rows and one slot of a lane, each in the low
// half of the dword its 2-byte LDS read returns (the high half is zero), are
// the B operand of one v_mfma_f32_16x16x32_f16 whose A operand is a 0/1
// routing matrix (lut_route in lut_device.h): the products add them over the
// slots and over four lanes at a time, in fp32, without vector-ALU adds or
// packing.  A
// short transposing butterfly over the remaining 16 lanes (fold_quads) leaves
// row (l >> 2) summed over the wave in lane l.  Each slice adds its row sums
// into one 64-bit word per row in the workspace (a contribution count plus a
// fixed-point sum, device-scope integer atomics); the lane whose atomic add
// completes the count holds the exact total, scales it by s_i, rounds to fp16,
// writes y and clears the word.  No barrier or counter is needed, results are
// bit-reproducible, and the workspace is zero again when the kernel ends.
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
// optional sign flips of the randomized variant: with four slots on one group
// tile every wave rotates its own activation fragment in registers, otherwise
// a few waves rotate each distinct block once and share it through LDS.
//
// S is the number of slots a workgroup holds tables for (1, 2 or 4): 64 KiB of
// LDS per pair of slots (S = 1 uses half of one pair's entries).  Building a
// slot's tables costs the same whatever the row count, so a launch with few
// slots (small k) takes fewer slots and more row tiles per workgroup.
//
// The fields the first loads depend on come first, as scalars, so that the
// launch preloads them into SGPRs (kernel-argument preloading; a by-value
// struct cannot be preloaded): a workgroup then issues its table operand and
// code loads without first waiting for an argument load.  packed0, codebooks0,
// plane_bytes0, n_rt0 and tpb0 are those of linear 0, which a single-linear
// launch uses; the other fields stay in the struct and are read after the
// table build.
template <int WAVES, int K, bool MULTI, int HB, int TPW, int S>
__global__ __launch_bounds__(64 * WAVES) void gemv_lut_kernel(const uint8_t* __restrict__ packed0,
                                                              const uint16_t* __restrict__ codebooks0,
                                                              const uint16_t* __restrict__ xin, int64_t plane_bytes0,
                                                              int n_rt0, int G, int slices, int n_slots, int tpb0,
                                                              LutArgs p) {
    static_assert(S == 1 || S == 2 || S == 4, "slots per workgroup");
    constexpr int NPAIR = S >= 2 ? S / 2 : 1;                      // 64 KiB table regions
    constexpr int H = S >= 2 ? 2 : 1;                              // slots per region
    // When K is a multiple of S every slot of the slice lies in one group tile.
    constexpr bool ONE_TILE = K % S == 0;
    // The rotating launch rotates in registers (each wave its own activation fragments) where four
    // slots share one group tile; elsewhere the distinct blocks are rotated once, by as many waves,
    // and shared through LDS.  Both give the bits of the standalone rotation.
    constexpr bool REG_ROT = HB > 0 && S == 4 && ONE_TILE;
    constexpr bool LDS_ROT = HB > 0 && !REG_ROT;
    constexpr int XS_SLOTS = ONE_TILE ? 1 : S;                     // staged slots (distinct group tiles)
    constexpr int XS_BYTES = LDS_ROT ? XS_SLOTS * TILE_GROUPS * GROUP * 2 : 0;   // rotated inputs, fp16
    __shared__ __align__(16) uint8_t lds[NPAIR * LUT_PAIR_BYTES + XS_BYTES + 16];
    uint16_t* xs = reinterpret_cast<uint16_t*>(lds + NPAIR * LUT_PAIR_BYTES);   // [staged slot][512]
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
    const uint8_t* const packed = MULTI ? p.lin[l].packed : packed0;
    const uint16_t* const codebooks = MULTI ? p.lin[l].codebooks : codebooks0;
    const int64_t plane_bytes = MULTI ? p.lin[l].plane_bytes : plane_bytes0;
    const int64_t n_rt = MULTI ? p.lin[l].n_rt : (int64_t)n_rt0;
    const int tiles_per_block = MULTI ? p.lin[l].tiles_per_block : tpb0;
    const int local = (int)blockIdx.x - (MULTI ? p.lin[l].wg_begin : 0);
    const int slice = local % slices;
    const int rb = local / slices;
    const int64_t t0 = (int64_t)rb * tiles_per_block;
    const int64_t t1 = t0 + tiles_per_block < n_rt ? t0 + tiles_per_block : n_rt;

    // slot s of this slice: q = slice*S + s -> group tile q / K, codebook q % K.
    // Every load below is unconditional (inactive slots, padding groups and
    // missing tiles read a valid address and the value is replaced by zero), so
    // the compiler can wait for exactly the loads a step needs.
    __amdgpu_buffer_rsrc_t slot_buf[S];
    bool slot_on[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int q = slice * S + s;
        slot_on[s] = q < n_slots;
        const int qq = slot_on[s] ? q : 0;
        slot_buf[s] = slot_rsrc(packed + (int64_t)(qq % K) * plane_bytes + (int64_t)(qq / K) * n_rt * TILE_BYTES,
                                n_rt * TILE_BYTES);
    }

    // ---- table operands first.  An item is a 32 x 32 block of one region:
    // codewords 32*cb .. +32 of both slots of pair `pair`, groups 32*gb .. +32.
    constexpr int ITEMS = 16 * NPAIR / WAVES;
    static_assert(ITEMS * WAVES == 16 * NPAIR, "items per wave");
    uint2 av[ITEMS][H], bv[ITEMS][H];
    uint64_t sw[ITEMS][H] = {};                                  // sign words (rotation in registers)
    bool bok[ITEMS][H];
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
        const int item = wave + u * WAVES;
        const int cb = (item >> 1) & 7, gb = item & 1, pair = item >> 4;
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int q = slice * S + 2 * pair + h;
            const int qq = q < n_slots ? q : 0;
            const int e0 = 4 * (lane >> 5);
            const int c = cb * 32 + (lane & 31);
            const int64_t g = (int64_t)(qq / K) * TILE_GROUPS + gb * 32 + (lane & 31);
            bok[u][h] = q < n_slots && g < G;
            const int64_t gc = g < G ? g : G - 1;
            av[u][h] = *reinterpret_cast<const uint2*>(codebooks + ((int64_t)(qq % K) * CODEWORDS + c) * GROUP + e0);
            // The activation fragment (raw when rotated in registers, below; read from LDS when the
            // rotation is staged there).  With one group tile the items of a wave share gb: one
            // fragment serves them all.
            if constexpr (!LDS_ROT) {
                if (!ONE_TILE || (u == 0 && h == 0)) {
                    bv[u][h] = *reinterpret_cast<const uint2*>(xin + gc * GROUP + e0);
                    // randomized rotation: the sign bits of the fragment's four inputs, bit n % 64 of word n / 64
                    if (REG_ROT && p.signs) sw[u][h] = p.signs[(gc * GROUP + e0) / 64];
                } else {
                    bv[u][h] = bv[0][0];
                    if (REG_ROT && p.signs) sw[u][h] = sw[0][0];
                }
            }
        }
    }
    // raw activation blocks of the staged rotation: staged slot s needs inputs 512*tile .. +512
    // (tile = q / K), i.e. 512 / HB blocks; wave w takes blocks w, w + WAVES, ...
    constexpr int BLK_PER_SLOT = LDS_ROT ? TILE_GROUPS * GROUP / HB : 1;
    constexpr int NBLK = XS_SLOTS * BLK_PER_SLOT;
    constexpr int BPW = (NBLK + WAVES - 1) / WAVES;
    constexpr int E = LDS_ROT ? HB / 64 : 1;
    float xv[BPW][E];
    bool xok[BPW];
    if constexpr (LDS_ROT) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int blk = wave + b * WAVES;
            const int sl = (blk < NBLK ? blk : 0) / BLK_PER_SLOT, j = (blk < NBLK ? blk : 0) % BLK_PER_SLOT;
            const int q = slice * S + sl;
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

    // The code stream is requested only once this wave's table operands have
    // arrived.  The operands are a few KB that every workgroup reads; requested
    // behind the code stream they would wait for a large part of it in the
    // memory queues, and every table build with them.  All waves of the
    // workgroup issue their operand loads first (barrier), then each wave waits
    // for its own.
    // routing matrices of the row sums (lane arithmetic only).  With 4 slots they are formed here,
    // while the operands are in flight, which measured faster; with fewer slots the compiler's
    // placement after the table build measured faster.
    half8_t route[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        route[q] = lut_route(q, lane);
        if constexpr (S == 4) {
            const uint4 rq = __builtin_bit_cast(uint4, route[q]);
            asm volatile("" ::"v"(rq.x), "v"(rq.y), "v"(rq.z), "v"(rq.w));
        }
    }
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int u = 0; u < ITEMS; ++u)
#pragma unroll
        for (int h = 0; h < H; ++h) {
            asm volatile("" ::"v"(av[u][h].x), "v"(av[u][h].y) : "memory");
            if (!LDS_ROT) asm volatile("" ::"v"(bv[u][h].x), "v"(bv[u][h].y) : "memory");
        }
    if constexpr (LDS_ROT) {
#pragma unroll
        for (int b = 0; b < BPW; ++b)
#pragma unroll
            for (int e = 0; e < E; ++e) asm volatile("" ::"v"(xv[b][e]) : "memory");
    }

    // ---- then the first code tile of every wave, in flight while the tables are
    // built; the other tiles are requested after the build (below), so that
    // workgroups still waiting for their operands are not queued behind them.
    uint4 codes[TPW][S];
    auto load_slot = [&](int u, int s) {
        const int64_t it = t0 + wave + (int64_t)u * WAVES;
        const uint32_t off = it < t1 ? (uint32_t)(it * TILE_BYTES) + lane * TILE_ROWS : NO_TILE;
        codes[u][s] = load_stream(slot_buf[s], slot_on[s] ? off : NO_TILE);
    };
    auto load_tile = [&](int u) {
#pragma unroll
        for (int s = 0; s < S; ++s) load_slot(u, s);
    };
    load_tile(0);
    if constexpr (LDS_ROT) {
#pragma unroll
        for (int b = 0; b < BPW; ++b) {
            const int blk = wave + b * WAVES;
            if (blk >= NBLK) continue;                          // uniform over the wave
            fwht_block<HB>(xv[b], lane);
#pragma unroll
            for (int e = 0; e < E; ++e) xs[blk * HB + e * 64 + lane] = xok[b] ? f2h(xv[b][e]) : (uint16_t)0;
        }
        __syncthreads();                                        // rotated inputs of every staged slot are in LDS
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            const int item = wave + u * WAVES;
            const int gb = item & 1, pair = item >> 4;
#pragma unroll
            for (int h = 0; h < H; ++h)
                bv[u][h] = *reinterpret_cast<const uint2*>(xs + (ONE_TILE ? 0 : 2 * pair + h) * (TILE_GROUPS * GROUP) +
                                                           (gb * 32 + (lane & 31)) * GROUP + 4 * (lane >> 5));
        }
    }
    if constexpr (REG_ROT) {
        // Each wave rotates the fragment it holds, in registers: a fragment is 256 inputs starting at a
        // multiple of 256, so it holds whole blocks, and fwht_operand gives them the bits of the
        // standalone rotation.  Fragments past the input are rotated from clamped inputs and then
        // zeroed with their groups (below); a block never straddles the end, d_in being a multiple of HB.
        const int pos = 8 * (lane & 7) + 4 * (lane >> 5);      // bit of the fragment's first input in its word
#pragma unroll
        for (int u = 0; u < ITEMS; ++u)
#pragma unroll
            for (int h = 0; h < H; ++h) {
                if (ONE_TILE && (u != 0 || h != 0)) {
                    bv[u][h] = bv[0][0];
                    continue;
                }
                const uint2 raw = bv[u][h];
                float v[4] = {h2f((uint16_t)(raw.x & 0xFFFF)), h2f((uint16_t)(raw.x >> 16)),
                              h2f((uint16_t)(raw.y & 0xFFFF)), h2f((uint16_t)(raw.y >> 16))};
                if (p.signs) {                                  // eps = -1 where the bit is set
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if ((sw[u][h] >> (pos + r)) & 1ull) v[r] = -v[r];
                }
                fwht_operand<(HB > 0 ? HB : 64)>(v, lane);
                bv[u][h] = make_uint2((uint32_t)f2h(v[0]) | ((uint32_t)f2h(v[1]) << 16),
                                      (uint32_t)f2h(v[2]) | ((uint32_t)f2h(v[3]) << 16));
            }
    }
#pragma unroll
    for (int u = 0; u < ITEMS; ++u)
#pragma unroll
        for (int h = 0; h < H; ++h) {
            if (!bok[u][h]) bv[u][h] = make_uint2(0u, 0u);     // zero activation -> zero table entries
        }

    // ---- tables: entry (slot s, codeword c, lane l) at byte (s/2)*64K + c*256 + l*4 + 2*(s%2)
#pragma unroll
    for (int u = 0; u < ITEMS; ++u) {
        const int item = wave + u * WAVES;
        const int pair = item >> 4, cb = (item >> 1) & 7, gb = item & 1;
        floatx16_t t[H];
#pragma unroll
        for (int h = 0; h < H; ++h) {
#pragma unroll
            for (int r = 0; r < 16; ++r) t[h][r] = 0.f;
            t[h] = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(half4_t, av[u][h]),
                                                        __builtin_bit_cast(half4_t, bv[u][h]), t[h], 0, 0, 0);
        }
        const int gl = gb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int c = cb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            uint8_t* dst = lds + pair * LUT_PAIR_BYTES + c * 256 + gl * 4;
            if constexpr (H == 2) *reinterpret_cast<half2_t*>(dst) = half2_t{(_Float16)t[0][r], (_Float16)t[H - 1][r]};
            else *reinterpret_cast<_Float16*>(dst) = (_Float16)t[0][r];
        }
    }
    __syncthreads();
    // with 2 or 4 slots, tile u + 1 is requested from inside tile u's lookups (below)
    if constexpr (S == 1) {
#pragma unroll
        for (int u = 1; u < TPW; ++u) load_tile(u);
    }

    const LutLinear L = p.lin[MULTI ? l : 0];
    // scales of the rows this lane may finish (needed only at the end; clamped)
    uint16_t row_scale[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int64_t row = (t0 + wave + (int64_t)u * WAVES) * TILE_ROWS + (lane >> 2);
        row_scale[u] = L.scales[row < L.d_out ? row : L.d_out - 1];
    }

    uint32_t base[S];
#pragma unroll
    for (int s = 0; s < S; ++s) base[s] = (uint32_t)(lane * 4 + 2 * (s & 1)) | ((uint32_t)(s >> 1) << 16);
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
        // per row quad q and slot pair: the entries (4 rows x the pair's slots) of this lane in the
        // fp16 halves of the B operand; one product routes them into D (lut_route)
        floatx4_t d = {0.f, 0.f, 0.f, 0.f};
        // (row quad q, slot sl) pairs in q-major order; the zero-extended 2-byte reads are the B dwords
        // (entry in the low half, zero above)
        auto read_pair = [&](int n, uint32_t (&e)[4]) {
            const int q = n / S, sl = n % S;
            const uint4& c = codes[u][sl];
            const uint32_t w = q == 0 ? c.x : q == 1 ? c.y : q == 2 ? c.z : c.w;
#pragma unroll
            for (int m = 0; m < 4; ++m) e[m] = *reinterpret_cast<const uint16_t*>(lds + lut_addr(w, base[sl], m));
        };
        constexpr int NP = 4 * S;
        if constexpr (S == 1) {
#pragma unroll
            for (int n = 0; n < NP; ++n) {
                uint32_t e[4];
                read_pair(n, e);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(route[n], __builtin_bit_cast(half8_t, make_uint4(e[0], e[1], e[2], e[3])),
                                                           d, 0, 0, 0);
            }
        } else {
            // Software pipeline: the reads of pair n + LA go out before the product of pair n (the
            // scheduling barriers keep that order), so a wave keeps 8 reads in flight instead of
            // draining them every two products; same products in the same order.  The next tile's
            // slots are requested from here, half after 3/8 and half after 11/16 of the products.
            constexpr int LA = 2;
            uint32_t e[LA + 1][4];
#pragma unroll
            for (int n = 0; n < LA; ++n) read_pair(n, e[n]);
#pragma unroll
            for (int n = 0; n < NP; ++n) {
                if (n + LA < NP) read_pair(n + LA, e[(n + LA) % (LA + 1)]);
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t (&cur)[4] = e[n % (LA + 1)];
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(route[n / S],
                                                           __builtin_bit_cast(half8_t, make_uint4(cur[0], cur[1], cur[2], cur[3])), d, 0, 0, 0);
                if (u + 1 < TPW) {
#pragma unroll
                    for (int sl = 0; sl < S; ++sl)
                        if (n == (sl < (S + 1) / 2 ? (6 * NP) / 16 : (11 * NP) / 16)) load_slot(u + 1, sl);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const float sum = fold_quads(d, lane);
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

// Slots per workgroup for one linear: as many as k (1, 2, then 4), more when
// the slices would exceed what a row's counted sum allows.  At k = 1 an input
// of 12 or more group tiles (6144 inputs) takes 2: half the slices, one row
// tile per wave on 4096 rows instead of two, and a tall layer fits one round
// of workgroups (4096x14336 5.3 -> 4.9 us, 14336x14336 13.0 -> 8.3 us; at 5120
// inputs even, at 4096 one slot is 0.1-0.2 us faster).  With 4 slots, a
// linear too small to give every wave of a workgroup a row tile (fewer tiles
// per workgroup than waves) takes 2: the 4-slot table build would otherwise
// sit on the critical path of half-idle workgroups (measured on 4096x4096 at
// k = 3 and 4: 5.9 -> 5.1 and 5.3 us).  A row's bits depend on this choice
// only, so it is made per linear, as if the linear ran alone.
static int lut_slots_for(int64_t n_gt, int k, int64_t n_rt) {
    int S = k <= 1 ? (n_gt >= 12 ? 2 : 1) : (k == 2 ? 2 : 4);
    if (S == 4 && k <= 4) {
        const int slices4 = lut_slices(n_gt, k, 4);
        const int64_t rb = LUT_CUS / slices4 >= 1 ? LUT_CUS / slices4 : 1;
        if ((n_rt + rb - 1) / rb < LUT_WAVES && lut_slices(n_gt, k, 2) <= LUT_MAX_SLICES) S = 2;
    }
    // k = 3 on long inputs: 2 slots when that plan still fits one round of workgroups (with four row
    // tiles per wave).  4096x14336 8.1 -> 7.7 us; where it would need a second round (8192x14336) it is
    // far slower, and at k = 4 the same rule was mixed (4096x14336 9.1 -> 9.7 us), so k = 4 keeps 4.
    if (k == 3 && S == 4 && n_gt >= 16) {
        const int sl2 = lut_slices(n_gt, k, 2);
        const int64_t per_wg = (int64_t)LUT_WAVES * LUT_TILES_PER_WAVE_BIG;
        if (sl2 <= LUT_MAX_SLICES && (n_rt + per_wg - 1) / per_wg * sl2 <= LUT_CUS) S = 2;
    }
    while (S < 4 && lut_slices(n_gt, k, S) > LUT_MAX_SLICES) S *= 2;
    return S;
}

#define AQD_LUT_ARGS a.lin[0].packed, a.lin[0].codebooks, a.x, a.lin[0].plane_bytes, (int)a.lin[0].n_rt, (int)a.G, \
                     a.slices, a.n_slots, a.lin[0].tiles_per_block, a

template <bool MULTI, int HB, int TPW, int S>
static void launch_kl(int k, dim3 gd, dim3 bd, hipStream_t s, const LutArgs& a) {
    switch (k) {
        case 1: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 1, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 2: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 2, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 3: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 3, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 4: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 4, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 5: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 5, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 6: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 6, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        case 7: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 7, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
        default: hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 8, MULTI, HB, TPW, S>), gd, bd, 0, s, AQD_LUT_ARGS); break;
    }
}

// S = 1 only occurs at k = 1 and S = 2 only at k <= 4 (lut_slots_for), so only
// those instantiations exist.
template <bool MULTI, int HB, int TPW>
static void launch_k(int k, int S, dim3 gd, dim3 bd, hipStream_t s, const LutArgs& a) {
    if (S == 1) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 1, MULTI, HB, TPW, 1>), gd, bd, 0, s, AQD_LUT_ARGS);
    else if (S == 2 && k == 1) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 1, MULTI, HB, TPW, 2>), gd, bd, 0, s, AQD_LUT_ARGS);
    else if (S == 2 && k == 2) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 2, MULTI, HB, TPW, 2>), gd, bd, 0, s, AQD_LUT_ARGS);
    else if (S == 2 && k == 3) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 3, MULTI, HB, TPW, 2>), gd, bd, 0, s, AQD_LUT_ARGS);
    else if (S == 2) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES, 4, MULTI, HB, TPW, 2>), gd, bd, 0, s, AQD_LUT_ARGS);
    else launch_kl<MULTI, HB, TPW, 4>(k, gd, bd, s, a);
}
#undef AQD_LUT_ARGS

template <bool MULTI, int HB>
static void launch_tpw(int tpw, int k, int S, dim3 gd, dim3 bd, hipStream_t s, const LutArgs& a) {
    if (tpw == LUT_TILES_PER_WAVE_BIG) launch_k<MULTI, HB, LUT_TILES_PER_WAVE_BIG>(k, S, gd, bd, s, a);
    else launch_k<MULTI, HB, LUT_TILES_PER_WAVE>(k, S, gd, bd, s, a);
}

// Single-linear launches whose plan leaves at most 8 row tiles per workgroup (S <= 2, two tiles per
// wave): the same plan in 8-wave workgroups.  Every tile and sum is as in the 16-wave launch, so are the
// bits; half the waves to launch and to wait for at the table barrier (4096x4096 k = 1 / 2: 3.78 / 4.26
// -> 3.57 / 3.97 us; 1024 and 2048 rows alike).
#define AQD_LUT_ARGS8 a.lin[0].packed, a.lin[0].codebooks, a.x, a.lin[0].plane_bytes, (int)a.lin[0].n_rt, \
                      (int)a.G, a.slices, a.n_slots, a.lin[0].tiles_per_block, a
template <int HB>
static void launch_w8(int k, int S, dim3 gd, hipStream_t s, const LutArgs& a) {
    const dim3 bd(64 * LUT_WAVES_SMALL);
    constexpr int T = LUT_TILES_PER_WAVE;
    if (S == 1) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES_SMALL, 1, false, HB, T, 1>), gd, bd, 0, s, AQD_LUT_ARGS8);
    else if (k == 1) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES_SMALL, 1, false, HB, T, 2>), gd, bd, 0, s, AQD_LUT_ARGS8);
    else if (k == 2) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES_SMALL, 2, false, HB, T, 2>), gd, bd, 0, s, AQD_LUT_ARGS8);
    else if (k == 3) hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES_SMALL, 3, false, HB, T, 2>), gd, bd, 0, s, AQD_LUT_ARGS8);
    else hipLaunchKernelGGL((gemv_lut_kernel<LUT_WAVES_SMALL, 4, false, HB, T, 2>), gd, bd, 0, s, AQD_LUT_ARGS8);
}
#undef AQD_LUT_ARGS8

// One launch over linears that share S; acc[i] is linear i's counted row words.
static hipError_t launch_lut_group(const LutLinearRef* lins, unsigned long long* const* acc, int n, int k, int S,
                                   const uint16_t* x, int64_t d_in, hipStream_t s, int rotate_block,
                                   const uint8_t* signs) {
    const int64_t G = d_in / GROUP;
    const int64_t n_gt = (G + TILE_GROUPS - 1) / TILE_GROUPS;
    LutArgs a = {};
    a.x = x;
    a.signs = rotate_block ? reinterpret_cast<const uint64_t*>(signs) : nullptr;
    a.G = G;
    a.n_gt = n_gt;
    a.k = k;
    a.n_slots = (int)((int64_t)k * n_gt);
    a.slices = lut_slices(n_gt, k, S);
    int64_t n_rt[LUT_MAX_GROUP];
    int tpb[LUT_MAX_GROUP], blocks[LUT_MAX_GROUP];
    for (int i = 0; i < n; ++i) {
        a.lin[i].packed = lins[i].packed;
        a.lin[i].codebooks = lins[i].codebooks;
        a.lin[i].scales = lins[i].scales;
        a.lin[i].y = lins[i].y;
        a.lin[i].acc = acc[i];
        a.lin[i].d_out = lins[i].d_out;
        a.lin[i].n_rt = (lins[i].d_out + TILE_ROWS - 1) / TILE_ROWS;
        a.lin[i].plane_bytes = a.lin[i].n_rt * n_gt * TILE_BYTES;
        n_rt[i] = a.lin[i].n_rt;
    }
    a.n_lin = n;
    // two row tiles per wave, or four when two would need more workgroups than CUs (a second round)
    const bool round4 = n == 1 && rotate_block == 0;   // the plain single-linear GEMV
    int tpw = LUT_TILES_PER_WAVE;
    lut_plan(n_rt, n, a.slices, tpw, tpb, blocks, round4);
    int64_t wgs = 0;
    for (int i = 0; i < n; ++i) wgs += (int64_t)a.slices * blocks[i];
    if (wgs > LUT_CUS) {
        tpw = LUT_TILES_PER_WAVE_BIG;
        lut_plan(n_rt, n, a.slices, tpw, tpb, blocks, round4);
    }
    int wg = 0;
    for (int i = 0; i < n; ++i) {
        a.lin[i].tiles_per_block = tpb[i];
        a.lin[i].wg_begin = wg;
        wg += a.slices * blocks[i];
    }
    const dim3 gd((unsigned)wg), bd(64 * LUT_WAVES);
    // one linear: the instantiation that takes every field its first loads need from the preloaded
    // leading arguments
    const bool one = n == 1;
    if (one && tpw == LUT_TILES_PER_WAVE && S <= 2 && k <= 4 && tpb[0] <= LUT_WAVES_SMALL) {
        if (rotate_block == 64) launch_w8<64>(k, S, gd, s, a);
        else if (rotate_block == 128) launch_w8<128>(k, S, gd, s, a);
        else if (rotate_block == 256) launch_w8<256>(k, S, gd, s, a);
        else launch_w8<0>(k, S, gd, s, a);
        return hipGetLastError();
    }
    if (rotate_block == 64) one ? launch_tpw<false, 64>(tpw, k, S, gd, bd, s, a) : launch_tpw<true, 64>(tpw, k, S, gd, bd, s, a);
    else if (rotate_block == 128)
        one ? launch_tpw<false, 128>(tpw, k, S, gd, bd, s, a) : launch_tpw<true, 128>(tpw, k, S, gd, bd, s, a);
    else if (rotate_block == 256)
        one ? launch_tpw<false, 256>(tpw, k, S, gd, bd, s, a) : launch_tpw<true, 256>(tpw, k, S, gd, bd, s, a);
    else one ? launch_tpw<false, 0>(tpw, k, S, gd, bd, s, a) : launch_tpw<true, 0>(tpw, k, S, gd, bd, s, a);
    return hipGetLastError();
}

hipError_t launch_gemv_lut_grouped(const LutLinearRef* lins, int n, int k, const uint16_t* x, int64_t d_in,
                                   void* ws, hipStream_t s, int rotate_block, const uint8_t* signs) {
    const int64_t n_gt = (d_in / GROUP + TILE_GROUPS - 1) / TILE_GROUPS;
    // each linear's row words sit at its place in the workspace, in argument order
    unsigned long long* acc[LUT_MAX_GROUP];
    int slots[LUT_MAX_GROUP];
    uint8_t* w = static_cast<uint8_t*>(ws);
    for (int i = 0; i < n; ++i) {
        acc[i] = reinterpret_cast<unsigned long long*>(w);
        w += acc_bytes(lins[i].d_out);
        slots[i] = lut_slots_for(n_gt, k, (lins[i].d_out + TILE_ROWS - 1) / TILE_ROWS);
    }
    // the linears that take the same slots per workgroup share one launch (all of them, in practice)
    for (int S = 1; S <= LUT_SLOTS; S *= 2) {
        LutLinearRef part[LUT_MAX_GROUP];
        unsigned long long* part_acc[LUT_MAX_GROUP];
        int m = 0;
        for (int i = 0; i < n; ++i)
            if (lins[i].d_out > 0 && slots[i] == S) {
                part[m] = lins[i];
                part_acc[m] = acc[i];
                ++m;
            }
        if (m == 0) continue;
        const hipError_t e = launch_lut_group(part, part_acc, m, k, S, x, d_in, s, rotate_block, signs);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_lut(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int k,
                           const uint16_t* x, uint16_t* y, const Geometry& g, void* ws, hipStream_t s) {
    const LutLinearRef one = {packed, codebooks, scales, y, g.d_out};
    return launch_gemv_lut_grouped(&one, 1, k, x, g.d_in, ws, s, 0, nullptr);
}

}  // namespace aqd
