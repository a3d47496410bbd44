#!/usr/bin/env python3
"""Writes fwd64_phases.h: the main loop of the 64-row-per-wave prefill
attention kernel (fwd64.hip) as one hand-scheduled inline-asm statement for
gfx950, plus the small helpers that reach its fixed registers.

Run from anywhere: ``python gen_fwd64.py`` rewrites fwd64_phases.h beside it
(the header is committed; a CPU test checks it matches this script).

Fixed registers (the compiler allocates none of them; every statement that
touches them names them as clobbered, and a CPU test checks the compiled
kernel never uses them outside these statements):

  a[64:191]   O^T accumulators, O[qh][db] = a[64 + 16*(4*qh+db) .. +15]
              (qh: query half of 32 rows, db: block of 32 head-dim columns)
  a[192:255]  Q^T MFMA operands, Q[qh][ds] = a[192 + 4*(8*qh+ds) .. +3]
              (ds: 16-column step of the head dimension)
  v[128:159]  SA: scores of query half 0 (key blocks 0, 1: 16 registers each)
  v[160:191]  SB: scores of query half 1 for even iterations
  v[192:223]  SC: scores of query half 1 for odd iterations
  v[224:239]  PA0, v[240:255] PA1: bf16 weights P of half 0 (even / odd)
  v[112:127]  PB: bf16 weights P of half 1
  v[96:111]   four K operand slots, v[80:95] four V operand slots
  v[64:79]    temporaries
  s[64:67]    buffer descriptor of the K tile being loaded, s[68:71] of V
  s[72:91]    loop bookkeeping

Iteration g of the loop (T[g]: the g-th key tile of the wave's group):
score phase: S(T[g+1]) = K Q^T on 32 MFMAs (both query halves share each K
fragment read from LDS) beside the softmax of T[g] for rows 32..63 and half
of the loads of K(T[g+2]) and V(T[g+1]), ending with the reads of the PV
phase's first V fragments; PV phase: O^T += V^T P^T for T[g] on 32 MFMAs
(both halves share each V fragment) beside the softmax of T[g+1] for rows
0..31, the other half of the loads and the next iteration's bookkeeping;
then a barrier.  What only some iterations need (masks, cache copies of the
tiles' own rows, the first tile of a run, the lower group's switch from the
light to the heavy block) sits behind one guard branch before each phase.
The VALU work is spread over the MFMA slots by an issue-cost model measured
on this part (an MFMA every 32 cycles leaves about 19 cycles of issue for
other instructions of the same wave).
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "fwd64_phases.h")

V_SA, V_SB, V_SC = 128, 160, 192
V_PA = (224, 240)
V_PB = 112
V_KF = 96
V_VF = 80
V_T = 64
A_O = 64
A_Q = 192

# temporaries (v[64:79])
T_MX0, T_MX1 = V_T + 0, V_T + 1     # row-max chains / permlane pair
T_TS = V_T + 0                      # a half-tile's sum of weights (the max chains reuse it)
T_THR = V_T + 2                     # m + 8
T_MNEW = V_T + 3
T_ALPHA = V_T + 4                   # rescale factor (kept to the end of the phase)
T_NINF = V_T + 5                    # -inf
T_VDD = V_T + 6                     # vd + R0 - 64 t (general diagonal mask)
T_INV = (V_T + 6, V_T + 7)          # 1 / row sums of the light block's halves (its store)
T_RS = list(range(V_T + 8, V_T + 16))  # weights in flight; O-rescale pipeline

# scalar registers of the loop.  Pairs alternate with the iteration's
# parity: iteration g of parity par = g % 2 reads T[g] from S_TT[par] and
# T[g+1] from S_TT[1 - par], so T[g+1] is already in place for g + 1.
S_VK = 64          # s[64:67] K descriptor
S_VV = 68          # s[68:71] V descriptor
S_G = 72           # iteration
S_TT = (73, 74)    # tiles T[g], T[g+1]
S_T2 = 75          # tile whose K is loaded in the iteration (T[g+2])
S_BB = (76, 77)    # blocks of T[g], T[g+1]
S_KK = (78, 79)    # softmax kinds: of T[g] (score phase), of T[g+1] (PV phase)
S_OO = (80, 92)    # olive flags (O holds data) of the score phase, of the PV phase
S_FLAG = 81
S_M0SAVE = 82
S_X, S_Y = 83, 84               # scratch
S_CB = 88          # s[88:91] cache-store descriptor
S_SPEC = 93        # nonzero: the iteration takes the out-of-line middle part
S_CS = 94          # score-phase variant: 0 the common one (all keys of T[g] visible)
S_CP = 95          # PV-phase variant: 0 the common one
S_NX, S_NY, S_NZ = 96, 97, 98   # scratch of the next iteration's bookkeeping
NUM_SGPR_FIXED = list(range(64, 99))


def roles(par):
    """Registers of an iteration of parity par."""
    return dict(T0=S_TT[par], T1=S_TT[1 - par], B0=S_BB[par], B1=S_BB[1 - par],
                KS=S_KK[par], KP=S_KK[1 - par], OS=S_OO[par], OP=S_OO[1 - par])


K_SLOT_BYTES = 16384                # one 64 x 128 bf16 tile
V_OFF = 32768                       # V ring after the K ring (per group)
LOOKAHEAD = 3                       # operand fragments in flight
ROWSTEP_LOADS = 8                   # global-to-LDS loads per wave and tile
MINIT = "0xf149f2ca"                # -1e30: running max before the first tile

MFMA = "v_mfma_f32_32x32x16_bf16"


def vr(a, n=1):
    return "v%d" % a if n == 1 else "v[%d:%d]" % (a, a + n - 1)


def ar(a, n=1):
    return "a%d" % a if n == 1 else "a[%d:%d]" % (a, a + n - 1)


def sr(a, n=1):
    return "s%d" % a if n == 1 else "s[%d:%d]" % (a, a + n - 1)


def s_bank(par):
    """Score registers of half 1 for iteration parity par."""
    return V_SB if par == 0 else V_SC


# ------------------------------------------------------------------ softmax
# out-of-line blocks of the loop (the exact path of the softmax), emitted
# after the loop's other out-of-line parts
RARE = []
# per-lane partial sum of one half-tile's weights above which the exact path
# runs: 2^16 (also catches inf and NaN)
TS_LIMIT = "0x47800000"


def p_loop(sbase, pbase, m):
    """p = 2^(s c - m) for the 32 scores at sbase (kept intact), through the
    rotating temporaries T_RS; P packed to bf16 pairs at pbase in the
    B-operand order of the PV MFMAs; T_TS = sum of the unrounded p in fp32
    (v_add: the dot-product form of the sum stalls beside the MFMAs on this
    part).  Every exp result is read at least two instructions after the
    exp (transcendental results need a wait state)."""
    R = T_RS
    groups = []

    def pack(k):
        a, b = R[(2 * k) % len(R)], R[(2 * k + 1) % len(R)]
        out = [["v_cvt_pk_bf16_f32 %s, %s, %s" % (vr(pbase + k), vr(a), vr(b))]]
        if k == 0:
            out.append(["v_add_f32 %s, %s, %s" % (vr(T_TS), vr(a), vr(b))])
        else:
            out += [["v_add_f32 %s, %s, %s" % (vr(T_TS), vr(T_TS), vr(a))],
                    ["v_add_f32 %s, %s, %s" % (vr(T_TS), vr(T_TS), vr(b))]]
        return out
    for i in range(32):
        groups.append(["v_fma_f32 %s, %s, %%[c], -%s" % (vr(R[i % len(R)]), vr(sbase + i), m)])
        if i >= 1:
            groups.append(["v_exp_f32 %s, %s" % (vr(R[(i - 1) % len(R)]), vr(R[(i - 1) % len(R)]))])
        if i >= 2 and (i - 2) % 2 == 1:
            groups += pack((i - 2) // 2)
    groups.append(["v_exp_f32 %s, %s" % (vr(R[31 % len(R)]), vr(R[31 % len(R)]))])
    groups.append(["s_nop 1"])
    groups += pack(15)
    return groups


def softmax_ops(qh, sbase, pbase, m, l, tag):
    """Online-softmax update of one query half over one 64-key tile.

    sbase: 32 score registers (key block 0: sbase..+15, block 1: +16..+31);
    the lane holds query row 32*qh + lane%32 and, in register r of key
    block kb, key 32*kb + 8*(r/4) + 4*(lane/32) + r%4.  Scores the causal
    mask hides are -inf already (mask_ops).  pbase: 16 registers of bf16
    pairs, P[k] = (p[2k], p[2k+1]) over the 32 scores in order, which is the
    B-operand order of the PV MFMAs.  m, l: the half's running max (exp2
    domain) and per-lane partial sum.

    The weights of any m are exact once O and l use the same m, so the
    common path takes p = 2^(s c - m) against the running max without
    the tile's max, and checks the lane's sum of the tile's 32 weights: at
    most 2^16 (no weight above it: O and l stay far from overflow) and the
    tile is done.  The first tile of a run has its row max taken before the
    phase (first_max, in the block that masks it), so the sum passes the
    bound only where a tile's scores pass m by more than about 11 (or m is
    still the initial -1e30); then the exact path out of line takes the
    tile's row max as in the textbook update, moves m when the max exceeds it by more than 8, sets S_FLAG and
    rescales l (O is rescaled at the end of the phase), recomputes the
    weights from the scores, which the common path left intact, and
    returns.

    Returns a list of groups; a group's instructions are emitted together.
    """
    back = ".Lsb%s_%%=" % tag
    exact = ".Lsx%s_%%=" % tag
    groups = p_loop(sbase, pbase, m)
    groups.append(["v_cmp_nge_f32 vcc, %s, %s" % (TS_LIMIT, vr(T_TS)),
                   "s_cbranch_vccnz %s" % exact,
                   "%s:" % back,
                   "v_add_f32 %s, %s, %s" % (l, l, vr(T_TS))])
    RARE.append(["%s:" % exact] + [x for grp in exact_ops(sbase, m, l, tag) + p_loop(sbase, pbase, m) for x in grp]
                + ["s_branch %s" % back])
    return groups


def rowmax_ops(sbase):
    """T_MX0 = c * (row max of the tile's 32 scores and the lane partner's):
    two v_max3 chains and one v_permlane32_swap."""
    groups = []
    live = list(range(32))
    chains = [live[:len(live) // 2], live[len(live) // 2:]]
    for ci, ch in enumerate(chains):
        t = T_MX0 + ci
        groups.append(["v_max3_f32 %s, %s, %s, %s" % (vr(t), vr(sbase + ch[0]), vr(sbase + ch[1]), vr(sbase + ch[2]))])
        rest = ch[3:]
        while len(rest) >= 2:
            groups.append(["v_max3_f32 %s, %s, %s, %s" % (vr(t), vr(t), vr(sbase + rest[0]), vr(sbase + rest[1]))])
            rest = rest[2:]
        if rest:
            groups.append(["v_max_f32 %s, %s, %s" % (vr(t), vr(t), vr(sbase + rest[0]))])
    groups.append(["v_max_f32 %s, %s, %s" % (vr(T_MX0), vr(T_MX0), vr(T_MX1)),
                   "v_mov_b32 %s, %s" % (vr(T_MX1), vr(T_MX0)),
                   "s_nop 1",
                   "v_permlane32_swap_b32 %s, %s" % (vr(T_MX0), vr(T_MX1)),
                   "s_nop 1",
                   "v_max_f32 %s, %s, %s" % (vr(T_MX0), vr(T_MX0), vr(T_MX1)),
                   # row max in the exp2 domain (c > 0)
                   "v_mul_f32 %s, %%[c], %s" % (vr(T_MX0), vr(T_MX0))])
    return groups


def first_max(sbase, m):
    """m = max(m, the tile's row max) for the first tile of a run, after its
    masks, where m is still the initial -1e30 and O and l are zero: the
    common path then keeps every weight of the tile at most 1.  (Past the
    last tile the olive flag reads as a run start too; the scores are all
    masked there and m stays.)"""
    return [x for grp in rowmax_ops(sbase) for x in grp] + ["v_max_f32 %s, %s, %s" % (m, m, vr(T_MX0))]


def exact_ops(sbase, m, l, tag):
    """The row max (rowmax_ops) and the lazy move of m: only when some
    lane's tile max exceeds it by more than 8, then l *= alpha now, O at the
    end of the phase (S_FLAG)."""
    groups = rowmax_ops(sbase)
    groups.append(["v_add_f32 %s, 0x41000000, %s" % (vr(T_THR), m)])
    lbl = ".Lnr%s_%%=" % tag
    groups.append(["v_cmp_gt_f32 vcc, %s, %s" % (vr(T_MX0), vr(T_THR)),
                   "s_cbranch_vccz %s" % lbl,
                   "v_max_f32 %s, %s, %s" % (vr(T_MNEW), m, vr(T_MX0)),
                   "v_sub_f32 %s, %s, %s" % (vr(T_ALPHA), m, vr(T_MNEW)),
                   "v_mov_b32 %s, %s" % (m, vr(T_MNEW)),
                   "v_exp_f32 %s, %s" % (vr(T_ALPHA), vr(T_ALPHA)),
                   "s_mov_b32 %s, 1" % sr(S_FLAG),
                   "s_nop 1",
                   "v_mul_f32 %s, %s, %s" % (l, l, vr(T_ALPHA)),
                   "%s:" % lbl])
    return groups


def mask_ops(kind, qh, sbase):
    """Scores of one query half over one tile that the causal mask hides, set
    to -inf before the phase's softmax (which then gives them weight 0 and
    leaves the running max alone): 'd' a partly hidden tile that starts at
    the wave's first row (key k > row q hidden, both relative to the tile /
    the half's first row; for half 0 key block 1 lies wholly above the
    diagonal), 'g' a partly hidden tile at any offset (v[T_VDD] = vd + R0 -
    64 t, see kind_of), 'm' every key.  Register layout as in softmax_ops."""
    out = ["v_mov_b32 %s, 0xff800000" % vr(T_NINF)]
    if kind == 'g':
        # any offset: key k hidden from row q when k - q > R0 - 64 t, i.e.
        # 32 (kb - qh) + 8 (r / 4) + r % 4 > vd + R0 - 64 t (v[T_VDD])
        for i in range(32):
            kb, r = i // 16, i % 16
            o = 32 * (kb - qh) + 8 * (r // 4) + r % 4
            out += ["v_cmp_gt_i32 vcc, %d, %s" % (o, vr(T_VDD)),
                    "v_cndmask_b32 %s, %s, %s, vcc" % (vr(sbase + i), vr(sbase + i), vr(T_NINF))]
        return out
    if kind == 'm':
        return out + ["v_mov_b32 %s, %s" % (vr(sbase + i), vr(T_NINF)) for i in range(32)]
    diag = range(16) if qh == 0 else range(16, 32)
    for i in diag:
        r = i % 16
        o = 8 * (r // 4) + r % 4
        out += ["v_cmp_gt_i32 vcc, %d, %%[vd]" % o,
                "v_cndmask_b32 %s, %s, %s, vcc" % (vr(sbase + i), vr(sbase + i), vr(T_NINF))]
    if qh == 0:
        out += ["v_mov_b32 %s, %s" % (vr(sbase + i), vr(T_NINF)) for i in range(16, 32)]
    return out


def o_rescale(qh, after_mfma, tag, olive):
    """O[qh] *= alpha when S_FLAG is set and the olive register is (O holds
    data)."""
    lbl = ".Lor%s_%%=" % tag
    out = ["s_and_b32 %s, %s, %s" % (sr(S_FLAG), sr(S_FLAG), sr(olive)),
           "s_cmp_eq_u32 %s, 0" % sr(S_FLAG),
           "s_cbranch_scc1 %s" % lbl]
    if after_mfma:
        # the phase's last MFMAs write these accumulators
        out += ["s_nop 7", "s_nop 7", "s_nop 7", "s_nop 7"]
    regs = list(range(A_O + 64 * qh, A_O + 64 * qh + 64))
    n = len(T_RS)
    for b in range(0, len(regs), n):
        chunk = regs[b:b + n]
        for t, a in zip(T_RS, chunk):
            out.append("v_accvgpr_read_b32 %s, %s" % (vr(t), ar(a)))
        for t, a in zip(T_RS, chunk):
            out.append("v_mul_f32 %s, %s, %s" % (vr(t), vr(t), vr(T_ALPHA)))
        for t, a in zip(T_RS, chunk):
            out.append("v_accvgpr_write_b32 %s, %s" % (ar(a), vr(t)))
    out += ["s_nop 2", "%s:" % lbl]
    return out


# ------------------------------------------------------------------ schedule
# Issue cost (cycles of the wave's issue beside a running MFMA) used to
# spread the softmax over the MFMA slots.
SLOT_BUDGET = 18


def cost(ins):
    op = ins.split()[0]
    if op.startswith("v_exp"):
        return 7
    if op.startswith("s_nop"):
        return int(ins.split()[1]) + 1
    if op.startswith("v_permlane"):
        return 4
    if op.startswith(("v_add_f32", "v_mul_f32", "v_mov_b32", "v_cndmask", "v_cmp", "v_max_f32", "v_sub_f32")):
        return 3
    if op.startswith("v_"):
        return 4
    if op.startswith(("ds_", "buffer_", "global_")):
        return 3
    if op.endswith(":"):
        return 0
    return 1


def gcost(g):
    return sum(cost(x) for x in g)


def schedule(mfmas, frag_reads, reads_per_frag, fillers, loadg, prefetched=False, tail=()):
    """Interleave: before every fourth MFMA (fragments f, f + 1) wait for
    their reads and issue the reads of fragments up to f + 3; load pair i =
    (before, after) goes around
    MFMA i; the filler
    groups (softmax) fill each MFMA slot up to SLOT_BUDGET issue cycles, in
    order (raised when the rest would not fit; what is left follows the last
    MFMA).  The first LOOKAHEAD fragments' reads open the phase unless the
    previous phase issued them (prefetched).  tail: reads of the next
    phase's first fragments, issued after the last wait (no older read is
    then outstanding)."""
    nfrag = len(frag_reads)
    out = []
    fi = 0
    if not prefetched:
        for f in range(min(LOOKAHEAD, nfrag)):
            out += frag_reads[f]
    issued = min(LOOKAHEAD, nfrag)
    last_wait = max(s for s in range(len(mfmas)) if s % 4 == 0)
    nslots = len(mfmas)
    load_at = {i: g for i, g in enumerate(loadg)}
    for s, (mf, f) in enumerate(mfmas):
        used = 0
        if s % 4 == 0:
            # one wait for the fragments of the next four MFMAs (f, f + 1),
            # then the reads of fragments up to f + 3 (their slots' previous
            # fragments, f - 2 and f - 1, have had their MFMAs issued)
            last = min(f + 1, nfrag - 1)
            pending = max(issued - 1 - last, 0) * reads_per_frag
            out.append("s_waitcnt lgkmcnt(%d)" % pending)
            used += 1
            while issued < nfrag and issued <= f + 3:
                out += frag_reads[issued]
                used += gcost(frag_reads[issued])
                issued += 1
            if s == last_wait:
                for grp in tail:
                    out += grp
                    used += gcost(grp)
        if s in load_at:
            out += load_at[s][0]
            used += gcost(load_at[s][0])
        out.append(mf)
        if s in load_at:
            out += load_at[s][1]
            used += gcost(load_at[s][1])
        left = nslots - s
        rest = sum(gcost(g) for g in fillers[fi:])
        target = max(SLOT_BUDGET, used + rest / left)
        placed = False
        while fi < len(fillers):
            c = gcost(fillers[fi])
            if placed and used + c > target:
                break
            out += fillers[fi]
            used += c
            fi += 1
            placed = True
    while fi < len(fillers):
        out += fillers[fi]
        fi += 1
    return out


# ------------------------------------------------------------------ phases
def loads(par, matrix):
    """This wave's eight 1 KB global-to-LDS loads of the next K or V tile,
    both issued in the score phase of iteration g: K(T[g+2]) into K slot
    g % 2, V(T[g+1]) into V slot (g+1) % 2 (their previous tiles were last
    read before the previous interval's barrier).  Instruction i fills LDS
    block 2*i + wsub of the slot from the tile's buffer descriptor +
    %[fk<i>] (rows 8*i + 4*wsub + lane/16); rows past the sequence are out
    of the descriptor's range and read as zero.  Loads 2j and 2j+1 share one
    M0 (= %[m0b] + offset of block 4j): the instruction offset 2048 of the
    odd one moves both its LDS and its memory address, so %[fk<odd>] holds
    the row offset less 2048.  Returns (before, after) pairs: the M0 write
    goes before an MFMA, the load after it (an LDS DMA needs one wait state
    after M0 is written)."""
    groups = []
    if matrix == 'k':
        slot_off = par * K_SLOT_BYTES
        desc = sr(S_VK, 4)
    else:
        slot_off = V_OFF + (1 - par) * K_SLOT_BYTES
        desc = sr(S_VV, 4)
    for i in range(ROWSTEP_LOADS):
        if i % 2 == 0:
            groups.append((["s_add_u32 m0, %%[m0b], %d" % (slot_off + 2048 * i)],
                           ["buffer_load_dwordx4 %%[fk%d], %s, 0 offen lds" % (i, desc)]))
        else:
            groups.append(([], ["buffer_load_dwordx4 %%[fk%d], %s, 0 offen offset:2048 lds" % (i, desc)]))
    return groups


# of the iteration's 16 loads, the last PV_LOADS go out in the PV phase
# (before its bookkeeping moves the load descriptors on): the four waves
# then issue half as many loads at once, and the score phase half as many
# issue slots (8 of 16 measured best; all 16 in the PV phase is slower)
PV_LOADS = 8


def load_groups(par):
    """The iteration's load groups, pairs sharing an M0 together: K0 K1 V0 V1
    K2 K3 ..."""
    k_l, v_l = loads(par, 'k'), loads(par, 'v')
    return [x for j in range(0, ROWSTEP_LOADS, 2) for x in (k_l[j], k_l[j + 1], v_l[j], v_l[j + 1])]


def light_store_groups():
    """The lower group's finished light block, stored from O during the
    heavy block's first score phase (O is free until that iteration's PV
    phase): per lane 1 / (own + partner row sum) for each half, then per
    block of 16 accumulators: read, scale, pack to bf16, one
    v_permlane32_swap per register pair (each lane then holds 8 consecutive
    columns: those of column group 2 cp + lane/32) and two 16-byte buffer
    stores through the output descriptor, built in S_CB, whose range ends
    at the sequence's last row.  Uses the V operand slots (idle in a score
    phase) and T_INV, T_MNEW (within one group)."""
    t = T_MNEW
    groups = [["s_mov_b32 %s, %%[olo]" % sr(S_CB), "s_mov_b32 %s, %%[ohi]" % sr(S_CB + 1),
               "s_mov_b32 %s, %%[onrec]" % sr(S_CB + 2), "s_mov_b32 %s, 0x20000" % sr(S_CB + 3)]]
    for qh, l in ((0, "%[l0n]"), (1, "%[l1n]")):
        inv = T_INV[qh]
        groups.append(["v_mov_b32 %s, %s" % (vr(inv), l), "v_mov_b32 %s, %s" % (vr(t), l), "s_nop 1",
                       "v_permlane32_swap_b32 %s, %s" % (vr(inv), vr(t)), "s_nop 1",
                       "v_add_f32 %s, %s, %s" % (vr(inv), vr(inv), vr(t)),
                       "v_rcp_f32 %s, %s" % (vr(inv), vr(inv)), "s_nop 1"])
    for qh in range(2):
        for db in range(4):
            o = A_O + 16 * (4 * qh + db)
            groups.append(["v_accvgpr_read_b32 %s, %s" % (vr(V_VF + i), ar(o + i)) for i in range(8)])
            groups.append(["v_accvgpr_read_b32 %s, %s" % (vr(V_VF + i), ar(o + i)) for i in range(8, 16)])
            groups.append(["v_mul_f32 %s, %s, %s" % (vr(V_VF + i), vr(T_INV[qh]), vr(V_VF + i)) for i in range(8)])
            groups.append(["v_mul_f32 %s, %s, %s" % (vr(V_VF + i), vr(T_INV[qh]), vr(V_VF + i)) for i in range(8, 16)])
            groups.append(["v_cvt_pk_bf16_f32 %s, %s, %s" % (vr(V_VF + k), vr(V_VF + 2 * k), vr(V_VF + 2 * k + 1))
                           for k in range(8)])
            groups.append(["s_nop 1",
                           "v_permlane32_swap_b32 %s, %s" % (vr(V_VF + 0), vr(V_VF + 2)),
                           "v_permlane32_swap_b32 %s, %s" % (vr(V_VF + 1), vr(V_VF + 3)),
                           "v_permlane32_swap_b32 %s, %s" % (vr(V_VF + 4), vr(V_VF + 6)),
                           "v_permlane32_swap_b32 %s, %s" % (vr(V_VF + 5), vr(V_VF + 7)),
                           "s_nop 1",
                           "buffer_store_dwordx4 %s, %%[oo%d], %s, 0 offen offset:%d" % (vr(V_VF, 4), qh, sr(S_CB, 4), 64 * db),
                           "buffer_store_dwordx4 %s, %%[oo%d], %s, 0 offen offset:%d" % (vr(V_VF + 4, 4), qh, sr(S_CB, 4), 64 * db + 32),
                           "s_nop 1"])
    return groups


def o_zero_ops():
    """O = 0 by eight MFMAs with zero operands (T_RS[0:4]) and C = 0."""
    z = vr(T_RS[0], 4)
    return (["v_mov_b32 %s, 0" % vr(T_RS[i]) for i in range(4)] + ["s_nop 4"] +
            ["%s %s, %s, %s, 0" % (MFMA, ar(A_O + 16 * i, 16), z, z) for i in range(8)])


def score_phase(par, tag, store=False):
    """Score phase of an iteration of parity par: S(T[g+1]) beside
    softmax(T[g], half 1), loads of K(T[g+2]) and V(T[g+1]) (descriptors
    S_VK, S_VV).  In the last iteration T[g+1] does not exist: its K slot
    holds a refilled tile and the scores go unused.  store: the lower
    group's first heavy iteration, which also stores the light block from O
    and then zeroes O for the heavy block's first PV phase."""
    body = ["v_mov_b32 %s, 0xff800000" % vr(T_NINF),
            "s_mov_b32 %s, 0" % sr(S_FLAG)]
    fill = softmax_ops(1, s_bank(par), V_PB, "%[m1v]", "%[l1v]", tag + "h1")
    if store:
        fill = interleave(fill, light_store_groups())
    loadg = load_groups(par)[:len(load_groups(par)) - PV_LOADS]
    kslot = (1 - par) * K_SLOT_BYTES          # K(T[g+1]) in slot (g+1) % 2
    nb = s_bank(1 - par)                      # half-1 scores of T[g+1]
    frag_reads = []
    mfmas = []
    for ds in range(8):
        for kb in range(2):
            f = 2 * ds + kb
            slot = V_KF + 4 * (f % 4)
            off = kslot + 128 * (ds >> 2) + kb * 32 * 256
            frag_reads.append(["ds_read_b128 %s, %%[kb%d] offset:%d" % (vr(slot, 4), ds & 3, off)])
            for qh in range(2):
                dst = (V_SA if qh == 0 else nb) + 16 * kb
                src_c = "0" if ds == 0 else vr(dst, 16)
                mfmas.append(("%s %s, %s, %s, %s" % (MFMA, vr(dst, 16), vr(slot, 4),
                                                     ar(A_Q + 4 * (8 * qh + ds), 4), src_c), f))
    # the PV phase's first V fragments (V(T[g]) is in LDS since the last
    # barrier; the V slots are idle in this phase, but the store variant
    # uses them as temporaries until its end): the PV phase starts without
    # waiting out a read's latency
    hoisted = pv_frag_reads(par)[:LOOKAHEAD]
    body += schedule(mfmas, frag_reads, 1, fill, loadg, tail=() if store else hoisted)
    body += o_rescale(1, after_mfma=False, tag=tag, olive=roles(par)["OS"])
    if store:
        # the PV MFMAs accumulate into O next
        body += ["s_nop 2"] + o_zero_ops() + ["s_nop 7", "s_nop 7"]
        for grp in hoisted:
            body += grp
    return body


def score_phase_last(par, tag):
    """Score phase of the group's last iteration: no T[g+1] to score and no
    tile to load, only the softmax of T[g] for rows 32..63 and, at the end,
    the reads of the PV phase's first V fragments."""
    body = ["v_mov_b32 %s, 0xff800000" % vr(T_NINF),
            "s_mov_b32 %s, 0" % sr(S_FLAG)]
    for grp in softmax_ops(1, s_bank(par), V_PB, "%[m1v]", "%[l1v]", tag + "h1"):
        body += grp
    body += o_rescale(1, after_mfma=False, tag=tag, olive=roles(par)["OS"])
    for grp in pv_frag_reads(par)[:LOOKAHEAD]:
        body += grp
    return body


def pv_phase_last(par):
    """PV phase of the group's last iteration: the products of T[g] alone
    (there is no T[g+1] to take the softmax of, no tile to load and no next
    iteration to keep books for)."""
    frag_reads = pv_frag_reads(par)
    mfmas = []
    for gg in range(4):
        for db in range(4):
            f = 4 * gg + db
            slot = V_VF + 4 * (f % 4)
            for qh in range(2):
                o = A_O + 16 * (4 * qh + db)
                pb = (V_PA[par] if qh == 0 else V_PB) + 4 * gg
                mfmas.append(("%s %s, %s, %s, %s" % (MFMA, ar(o, 16), vr(slot, 4), vr(pb, 4), ar(o, 16)), f))
    return ["s_nop 1"] + schedule(mfmas, frag_reads, 2, [], [], prefetched=True)


def interleave(main, extra):
    """The groups of main with those of extra spread evenly among them."""
    if not main:
        return list(extra)
    out, n, k = [], len(main), len(extra)
    at = [((i + 1) * n) // (k + 1) for i in range(k)]
    j = 0
    for i, grp in enumerate(main):
        while j < k and at[j] <= i:
            out.append(extra[j])
            j += 1
        out.append(grp)
    out += extra[j:]
    return out


def pv_frag_reads(par):
    """LDS reads of the PV phase's V fragments (V(T[g]) in V slot g % 2):
    fragment f = 4 gg + db into V operand slot f % 4."""
    vslot = V_OFF + par * K_SLOT_BYTES
    out = []
    for gg in range(4):
        for db in range(4):
            f = 4 * gg + db
            slot = V_VF + 4 * (f % 4)
            off = vslot + 128 * (db >> 1) + 4096 * gg
            out.append(["ds_read_b64_tr_b16 %s, %%[vb%d] offset:%d" % (vr(slot, 2), db & 1, off),
                        "ds_read_b64_tr_b16 %s, %%[vb%d] offset:%d" % (vr(slot + 2, 2), db & 1, off + 2048)])
    return out


def pv_phase(par, has_pv, tag):
    """PV phase of an iteration of parity par: O += P(T[g]) V(T[g]) (if
    has_pv) beside softmax(T[g+1], half 0) and
    the scalar bookkeeping of iteration g + 1."""
    body = ["v_mov_b32 %s, 0xff800000" % vr(T_NINF),
            "s_mov_b32 %s, 0" % sr(S_FLAG)]
    fill = softmax_ops(0, V_SA, V_PA[1 - par], "%[m0v]", "%[l0v]", tag + "h0")
    fill = interleave(fill, book_fast(par))
    if has_pv:
        frag_reads = pv_frag_reads(par)
        mfmas = []
        for gg in range(4):
            for db in range(4):
                f = 4 * gg + db
                slot = V_VF + 4 * (f % 4)
                for qh in range(2):
                    o = A_O + 16 * (4 * qh + db)
                    pb = (V_PA[par] if qh == 0 else V_PB) + 4 * gg
                    mfmas.append(("%s %s, %s, %s, %s" % (MFMA, ar(o, 16), vr(slot, 4), vr(pb, 4), ar(o, 16)), f))
        body += ["s_nop 1"]   # the weights were written by VALU instructions
        lg = load_groups(par)
        pv_loads = lg[len(lg) - PV_LOADS:] if PV_LOADS else []
        sched = schedule(mfmas, frag_reads, 2, fill, pv_loads, prefetched=True)
        if pv_loads:
            # the loads read the descriptors before book_fast moves them on
            last_load = max(i for i, x in enumerate(sched) if x.startswith("buffer_load"))
            first_move = min(i for i, x in enumerate(sched) if x.startswith("s_add_u32 %s" % sr(S_VK))
                             or x.startswith("s_add_u32 %s" % sr(S_VV)))
            assert last_load < first_move, (last_load, first_move)
        body += sched
    else:
        # (the pre-loop iteration: its PV-phase loads before the bookkeeping)
        lg = load_groups(par)
        for before, after in (lg[len(lg) - PV_LOADS:] if PV_LOADS else []):
            body += before + ["s_nop 0"] + after
        for g in fill:
            body += g
    body += o_rescale(0, after_mfma=has_pv, tag=tag, olive=roles(par)["OP"])
    body += book_check(tag)
    return body


# ------------------------------------------------------------------ the loop
def tile_of(x, t, b, tmp=S_Y):
    """t = T[x], b = block of T[x]: light run (x < elo) or heavy run."""
    return ["s_cmp_lt_i32 %s, %%[elo]" % x,
            "s_cselect_b32 %s, 0, %%[jump]" % sr(tmp),
            "s_cselect_b32 %s, %%[blk0], %%[blk1]" % sr(b),
            "s_add_i32 %s, %s, %s" % (sr(t), x, sr(tmp))]


def kind_of(t, b, dst, tmp=S_Y):
    """dst = 0 if every row of the wave in block b sees every key of tile t,
    2 if none sees any, 1 otherwise.  The wave's first row sits at key
    position R0 = 128 b + %[r0p] (r0p: the keys before the sequence's first
    query, plus 64 wsub), so tiles below (R0 + 1) / 64 are wholly visible
    and tiles above (R0 + 63) / 64 wholly hidden (one tile in between when
    R0 is a multiple of 64, two otherwise)."""
    return ["s_lshl_b32 %s, %s, 7" % (sr(tmp), sr(b)),
            "s_add_i32 %s, %s, %%[r0p]" % (sr(tmp), sr(tmp)),
            "s_add_i32 %s, %s, 1" % (sr(tmp), sr(tmp)),         # R0 + 1
            "s_lshr_b32 %s, %s, 6" % (sr(dst), sr(tmp)),
            "s_cmp_lt_i32 %s, %s" % (sr(t), sr(dst)),
            "s_cselect_b32 %s, 0, 1" % sr(dst),
            "s_add_i32 %s, %s, 62" % (sr(tmp), sr(tmp)),        # R0 + 63
            "s_lshr_b32 %s, %s, 6" % (sr(tmp), sr(tmp)),
            "s_cmp_gt_i32 %s, %s" % (sr(t), sr(tmp)),
            "s_cselect_b32 %s, 2, %s" % (sr(dst), sr(dst))]


def descriptor(t, d, lo, hi, tmp=S_Y):
    """Buffer descriptor of tile t's rows: base + t * tile bytes, range to
    the end of the sequence's rows."""
    return ["s_mul_i32 %s, %s, %%[tileb]" % (sr(tmp), sr(t)),
            "s_add_u32 %s, %%[%s], %s" % (sr(d), lo, sr(tmp)),
            "s_addc_u32 %s, %%[%s], 0" % (sr(d + 1), hi),
            "s_sub_u32 %s, %%[nrec], %s" % (sr(d + 2), sr(tmp))]


def book_next(par):
    """Scalar state of iteration h = g + 1 (parity 1 - par), computed in the
    PV phase of iteration g as filler groups (each group keeps its own SCC
    uses): T[h+1] and its block and kind, the olive flag of h's PV phase,
    T[h+2] and the load descriptors, the flag of the out-of-line middle part
    and the phase variant codes.  T[h], its block and kind and the olive flag
    of h's score phase are g's T[g+1] values, already in h's registers."""
    r = roles(1 - par)
    g = sr(S_G)
    NX, NY, NZ = sr(S_NX), sr(S_NY), sr(S_NZ)
    T0, T1, B0, B1 = sr(r["T0"]), sr(r["T1"]), sr(r["B0"]), sr(r["B1"])
    KS, KP, OP = sr(r["KS"]), sr(r["KP"]), sr(r["OP"])
    return [
        # T[h+1] = T[g+2], its block
        ["s_add_i32 %s, %s, 2" % (NX, g)] + tile_of(NX, r["T1"], r["B1"], tmp=S_NY),
        # its kind; 3 when it is past the wave's tiles
        kind_of(r["T1"], r["B1"], r["KP"], tmp=S_NZ),
        ["s_cmp_lt_i32 %s, %%[nmy]" % NX, "s_cselect_b32 %s, %s, 3" % (KP, KP)],
        # olive of h's PV phase: T[h+1] does not start a run
        ["s_cmp_eq_u32 %s, %%[elo]" % NX, "s_cselect_b32 %s, 0, 1" % OP,
         "s_cmp_eq_u32 %s, 0" % NX, "s_cselect_b32 %s, 0, %s" % (OP, OP)],
        # T[h+2], or T[h] again when there is none (the load refills a free slot)
        ["s_add_i32 %s, %s, 3" % (NY, g), "s_cmp_lt_i32 %s, %%[elo]" % NY,
         "s_cselect_b32 %s, 0, %%[jump]" % NZ, "s_add_i32 %s, %s, %s" % (sr(S_T2), NY, NZ),
         "s_cmp_lt_i32 %s, %%[nmy]" % NY, "s_cselect_b32 %s, %s, %s" % (sr(S_T2), sr(S_T2), T0)],
        descriptor(S_T2, S_VK, "kbl", "kbh", tmp=S_NY),
        # V of T[h+1], or of T[h] when there is no T[h+1]
        ["s_cmp_eq_u32 %s, 3" % KP, "s_cselect_b32 %s, %s, %s" % (NY, T0, T1)] +
        descriptor(S_NY, S_VV, "vbl", "vbh", tmp=S_NY),
        # rare parts: Q reload (h + 1 == gt), transition (h == gt), the light
        # block's store (h == gt + 1)
        ["s_add_i32 %s, %s, 2" % (NY, g), "s_cmp_eq_u32 %s, %%[gt]" % NY, "s_cselect_b32 %s, 1, 0" % sr(S_SPEC),
         "s_add_i32 %s, %s, 1" % (NY, g), "s_cmp_eq_u32 %s, %%[gt]" % NY,
         "s_cselect_b32 %s, 1, %s" % (sr(S_SPEC), sr(S_SPEC)),
         "s_cmp_eq_u32 %s, %%[gt]" % g, "s_cselect_b32 %s, 1, %s" % (sr(S_SPEC), sr(S_SPEC))],
        # ... or a cache copy of K(T[h+1]) or V(T[h]) (tiles of the wave's own block)
        ["s_lshr_b32 %s, %s, 1" % (NY, T1), "s_cmp_eq_u32 %s, %s" % (NY, B1), "s_cselect_b32 %s, 1, 0" % NY,
         "s_cmp_eq_u32 %s, 3" % KP, "s_cselect_b32 %s, 0, %s" % (NY, NY)],
        ["s_lshr_b32 %s, %s, 1" % (NZ, T0), "s_cmp_eq_u32 %s, %s" % (NZ, B0), "s_cselect_b32 %s, 1, 0" % NZ,
         "s_or_b32 %s, %s, %s" % (NY, NY, NZ), "s_cmp_eq_u32 %[copy], 0",
         "s_cselect_b32 %s, 0, %s" % (NY, NY), "s_or_b32 %s, %s, %s" % (sr(S_SPEC), sr(S_SPEC), NY)],
        # variant codes: masks needed (and for the PV phase, its products),
        # + 8 for the first tile of a run (its max starts the running max);
        # the score phase + 16 when there is no T[h+1] to score
        ["s_cmp_eq_u32 %s, 0" % sr(r["OS"]), "s_cselect_b32 %s, 8, 0" % NY, "s_or_b32 %s, %s, %s" % (sr(S_CS), KS, NY),
         "s_cmp_eq_u32 %s, 3" % KP, "s_cselect_b32 %s, 16, 0" % NY, "s_or_b32 %s, %s, %s" % (sr(S_CS), sr(S_CS), NY),
         "s_cmp_eq_u32 %s, 0" % OP, "s_cselect_b32 %s, 8, 0" % NY, "s_or_b32 %s, %s, %s" % (sr(S_CP), KP, NY)],
    ]


def book_fast(par):
    """The common case of book_next: iteration h = g + 1 lies inside the
    loop entry's window of iterations (%[wlom1] < h <= %[wlom1] + 1 +
    %[wwid]) where T[h], T[h+1], T[h+2] are consecutive tiles of one run,
    all below the wave's diagonal and the block's own tiles, and h + 1
    does not start a run: then T[h+1] = T[h] + 1 in the same block, kind 0,
    olive, the load descriptors move on by one tile, and no part of the
    iteration is out of line.  Always run; book_check redoes the whole of
    book_next when h is outside the window."""
    r = roles(1 - par)
    T0, T1, B0, B1 = sr(r["T0"]), sr(r["T1"]), sr(r["B0"]), sr(r["B1"])
    KP, OP = sr(r["KP"]), sr(r["OP"])
    out = [["s_add_i32 %s, %s, 1" % (T1, T0), "s_mov_b32 %s, %s" % (B1, B0)],
           ["s_mov_b32 %s, 0" % KP, "s_mov_b32 %s, 1" % OP]]
    for d in (S_VK, S_VV):
        out.append(["s_add_u32 %s, %s, %%[tileb]" % (sr(d), sr(d)),
                    "s_addc_u32 %s, %s, 0" % (sr(d + 1), sr(d + 1)),
                    "s_sub_u32 %s, %s, %%[tileb]" % (sr(d + 2), sr(d + 2))])
    out.append(["s_mov_b32 %s, 0" % sr(S_SPEC), "s_mov_b32 %s, 0" % sr(S_CS), "s_mov_b32 %s, 0" % sr(S_CP)])
    return out


def book_check(tag):
    """After the PV phase: h = g + 1 outside the window takes the whole
    book_next (out of line, book_slow)."""
    return ["s_sub_u32 %s, %s, %%[wlom1]" % (sr(S_NX), sr(S_G)),
            "s_cmp_gt_u32 %s, %%[wwid]" % sr(S_NX),
            "s_cbranch_scc1 .Lbk%s_%%=" % tag,
            ".Lbd%s_%%=:" % tag]


def book_slow(par, tag):
    out = [".Lbk%s_%%=:" % tag]
    for grp in book_next(par):
        out += grp
    return out + ["s_branch .Lbd%s_%%=" % tag]


def book_entry(par):
    """Scalar state of iteration g = S_G (parity par) on entry to the loop:
    T[g] (T[0] for the pre-loop iteration g = -1), its block, kind (3: no
    softmax) and score-phase olive flag, then the rest as the previous
    iteration's PV phase would have computed it."""
    r = roles(par)
    g = sr(S_G)
    out = ["s_max_i32 %s, %s, 0" % (sr(S_X), g)] + tile_of(sr(S_X), r["T0"], r["B0"])
    out += kind_of(r["T0"], r["B0"], r["KS"])
    out += ["s_cmp_lt_i32 %s, 0" % g, "s_cselect_b32 %s, 3, %s" % (sr(r["KS"]), sr(r["KS"])),
            "s_cmp_eq_u32 %s, %%[elo]" % g, "s_cselect_b32 %s, 0, 1" % sr(r["OS"]),
            "s_cmp_eq_u32 %s, 0" % g, "s_cselect_b32 %s, 0, %s" % (sr(r["OS"]), sr(r["OS"]))]
    out += ["s_add_i32 %s, %s, -1" % (g, g)]
    for grp in book_next(1 - par):
        out += grp
    out += ["s_add_i32 %s, %s, 1" % (g, g),
            # the pre-loop iteration has no PV phase (and may need no copy of V)
            "s_cmp_lt_i32 %s, 0" % g, "s_cselect_b32 %s, 4, 0" % sr(S_NY),
            "s_or_b32 %s, %s, %s" % (sr(S_CP), sr(S_CP), sr(S_NY)),
            "s_or_b32 %s, %s, %s" % (sr(S_SPEC), sr(S_SPEC), sr(S_NY))]
    return out


def cache_copy(par, matrix, tag):
    """Copy this wave's 32 rows (32 wsub + 4 i + lane/16, i < 8) of the K
    tile T[g+1] (K slot (g+1) % 2) or the V tile T[g] (V slot g % 2) from LDS
    to the cache.  Buffer stores through a descriptor whose range ends at the
    sequence's last row drop the rows past it."""
    r = roles(par)
    if matrix == 'k':
        slot_off, t, lo, hi = (1 - par) * K_SLOT_BYTES, r["T1"], "kcl", "kch"
    else:
        slot_off, t, lo, hi = V_OFF + par * K_SLOT_BYTES, r["T0"], "vcl", "vch"
    out = []
    regs = [V_VF + 4 * i for i in range(4)] + [V_KF + 4 * i for i in range(4)]
    for i in range(8):
        out.append("ds_read_b128 %s, %%[cl] offset:%d" % (vr(regs[i], 4), slot_off + 1024 * i))
    # descriptor of the sequence's cache rows of this K/V head (256 B each);
    # the tile's first row (64 t) and its 17th (+4 KB) as store offsets
    out += ["s_mov_b32 %s, %%[%s]" % (sr(S_CB), lo),
            "s_mov_b32 %s, %%[%s]" % (sr(S_CB + 1), hi),
            "s_lshl_b32 %s, %%[len], 8" % sr(S_CB + 2),
            "s_mov_b32 %s, 0x20000" % sr(S_CB + 3),
            "s_lshl_b32 %s, %s, 14" % (sr(S_X), sr(t)),
            "s_add_u32 %s, %s, 4096" % (sr(S_Y), sr(S_X)),
            "s_waitcnt lgkmcnt(0)"]
    for i in range(8):
        soff = sr(S_X) if i < 4 else sr(S_Y)
        coff = "%[coe]" if i % 2 == 0 else "%[coo]"
        out.append("buffer_store_dwordx4 %s, %s, %s, %s offen offset:%d nt"
                   % (vr(regs[i], 4), coff, sr(S_CB, 4), soff, 1024 * (i % 4)))
    return out


def q_reload():
    """The heavy block's Q rows into the Q registers (lower group, after the
    last light score tile); waited for by the interval's vmcnt(0)."""
    out = []
    for qh in range(2):
        for ds in range(8):
            out.append("global_load_dwordx4 %s, %%[qo%d], %%[qb] offset:%d" % (ar(A_Q + 4 * (8 * qh + ds), 4), qh, 32 * ds))
    return out


def lbl(name, par):
    return ".L%s_p%d_%%=" % (name, par)


def copy_part(par):
    """Cache copies of own rows: K(T[g+1]) and V(T[g]), both in LDS since the
    previous barrier (run when S_SPEC is set)."""
    L = lambda name: lbl(name, par)
    P = "p%d" % par
    r = roles(par)
    g = sr(S_G)
    return (["s_cmp_eq_u32 %s, 0" % sr(S_SPEC),
             "s_cbranch_scc1 %s" % L("nocv"),
             "s_cmp_eq_u32 %[copy], 0",
             "s_cbranch_scc1 %s" % L("nocv"),
             "s_cmp_eq_u32 %s, 3" % sr(r["KP"]),
             "s_cbranch_scc1 %s" % L("nock"),
             "s_lshr_b32 %s, %s, 1" % (sr(S_X), sr(r["T1"])),
             "s_cmp_eq_u32 %s, %s" % (sr(S_X), sr(r["B1"])),
             "s_cbranch_scc0 %s" % L("nock")] + cache_copy(par, 'k', P) + ["%s:" % L("nock"),
            "s_cmp_lt_i32 %s, 0" % g,
            "s_cbranch_scc1 %s" % L("nocv"),
            "s_lshr_b32 %s, %s, 1" % (sr(S_X), sr(r["T0"])),
            "s_cmp_eq_u32 %s, %s" % (sr(S_X), sr(r["B0"])),
            "s_cbranch_scc0 %s" % L("nocv")] + cache_copy(par, 'v', P) + ["%s:" % L("nocv")])


def diag_mask(qh, sbase, t, b, tag):
    """Masks of a partly hidden tile t of block b for query half qh: the
    'd' form when the tile starts at the wave's first row (R0 = 64 t), else
    the general one."""
    return ["s_lshl_b32 %s, %s, 7" % (sr(S_X), sr(b)),
            "s_add_i32 %s, %s, %%[r0p]" % (sr(S_X), sr(S_X)),
            "s_lshl_b32 %s, %s, 6" % (sr(S_Y), sr(t)),
            "s_sub_i32 %s, %s, %s" % (sr(S_X), sr(S_X), sr(S_Y)),
            "s_cmp_eq_u32 %s, 0" % sr(S_X),
            "s_cbranch_scc0 .Lmg%s_%%=" % tag] + mask_ops('d', qh, sbase) + [
            "s_branch .Lmd%s_%%=" % tag,
            ".Lmg%s_%%=:" % tag,
            "v_add_u32 %s, %s, %%[vd]" % (vr(T_VDD), sr(S_X))] + mask_ops('g', qh, sbase) + [
            ".Lmd%s_%%=:" % tag]


def score_mask_part(par):
    """Score phase of a tile T[g] that is not wholly visible (or of no tile:
    the pre-loop iteration): its half-1 scores are masked first."""
    L = lambda name: lbl(name, par)
    KS = sr(roles(par)["KS"])
    out = ["s_cmp_eq_u32 %s, 0" % sr(S_CS),
           "s_cbranch_scc1 %s" % L("smend"),
           "s_cmp_eq_u32 %s, 1" % KS,
           "s_cbranch_scc1 %s" % L("ssd"),
           "s_cmp_eq_u32 %s, 0" % KS,
           "s_cbranch_scc1 %s" % L("smend")]
    r = roles(par)
    out += mask_ops('m', 1, s_bank(par)) + ["s_branch %s" % L("smend"), "%s:" % L("ssd")]
    out += diag_mask(1, s_bank(par), r["T0"], r["B0"], "s%d" % par)
    # the first tile of a run starts the running max of half 1
    out += ["%s:" % L("smend"),
            "s_cmp_eq_u32 %s, 0" % sr(r["OS"]),
            "s_cbranch_scc0 %s" % L("snf")] + first_max(s_bank(par), "%[m1v]") + ["%s:" % L("snf")]
    # the lower group's first heavy iteration (g == gt + 1) takes the score
    # phase that also stores the light block; the group's last iteration
    # (no T[g+1]) the one without score products and loads
    out += [
            "s_add_i32 %s, %%[gt], 1" % sr(S_X),
            "s_cmp_eq_u32 %s, %s" % (sr(S_G), sr(S_X)),
            "s_cbranch_scc1 %s" % L("sst"),
            "s_cmp_eq_u32 %s, 3" % sr(r["KP"]),
            "s_cbranch_scc1 %s" % L("snm")]
    return out


def middle_part(par):
    """Between the phases (run when S_SPEC is set): the heavy block's Q after
    the last light score tile; at the last light tile the next tile's half-0
    softmax starts the heavy block's state (the light block's is kept for
    its store)."""
    L = lambda name: lbl(name, par)
    g = sr(S_G)
    out = ["s_cmp_eq_u32 %s, 0" % sr(S_SPEC),
           "s_cbranch_scc1 %s" % L("notr"),
           "s_add_i32 %s, %s, 1" % (sr(S_X), g),
           "s_cmp_eq_u32 %s, %%[gt]" % sr(S_X),
           "s_cbranch_scc0 %s" % L("noq")] + q_reload() + ["%s:" % L("noq")]
    # (the half-1 state of the light block is final after this score phase:
    # its row sum is kept for the store, and half 1 restarts with the next
    # tile; the bookkeeping window moves to the heavy run)
    out += ["s_cmp_eq_u32 %s, %%[gt]" % g,
            "s_cbranch_scc0 %s" % L("notr"),
            "v_mov_b32 %[m0n], %[m0v]",
            "v_mov_b32 %[l0n], %[l0v]",
            "v_mov_b32 %%[m0v], %s" % MINIT,
            "v_mov_b32 %[l0v], 0",
            "v_mov_b32 %[l1n], %[l1v]",
            "v_mov_b32 %%[m1v], %s" % MINIT,
            "v_mov_b32 %[l1v], 0",
            "s_mov_b32 %[wlom1], %[wlom1b]",
            "s_mov_b32 %[wwid], %[wwidb]",
            "%s:" % L("notr")]
    return out


def pv_mask_part(par):
    """PV phase when T[g+1] is not wholly visible (or missing): its half-0
    scores are masked first (the score phase's MFMAs wrote them: wait them
    out); the pre-loop iteration (g < 0) leaves for its phase without PV
    products."""
    L = lambda name: lbl(name, par)
    KP = sr(roles(par)["KP"])
    out = ["s_cmp_eq_u32 %s, 0" % sr(S_CP),
           "s_cbranch_scc1 %s" % L("pgo"),
           # the group's last iteration: no T[g+1], so no softmax and no loads
           "s_cmp_eq_u32 %s, 3" % KP,
           "s_cbranch_scc1 %s" % L("pnm"),
           "s_nop 7", "s_nop 7", "s_nop 7",
           "s_cmp_eq_u32 %s, 1" % KP,
           "s_cbranch_scc1 %s" % L("psd"),
           "s_cmp_eq_u32 %s, 0" % KP,
           "s_cbranch_scc1 %s" % L("psv")]
    r = roles(par)
    out += mask_ops('m', 0, V_SA) + ["s_branch %s" % L("psv"), "%s:" % L("psd")]
    out += diag_mask(0, V_SA, r["T1"], r["B1"], "p%d" % par)
    # the first tile of a run starts the running max of half 0
    out += ["%s:" % L("psv"),
            "s_cmp_eq_u32 %s, 0" % sr(r["OP"]),
            "s_cbranch_scc0 %s" % L("pnf")] + first_max(V_SA, "%[m0v]") + ["%s:" % L("pnf"),
            "s_cmp_lt_i32 %s, 0" % sr(S_G),
            "s_cbranch_scc1 %s" % L("pre")]
    return out


def body(par):
    """One iteration (parity par) for g = S_G, ending after its barrier.  The
    two phases exist once each; what differs between iterations (cache
    copies, masked scores, Q reload, transition) sits in line in two blocks,
    one before each phase, that the common iteration jumps over with one
    branch each: code met only on a few iterations then lies on the
    instruction fetch's sequential path instead of at distant targets that
    each cost a cold instruction-cache miss.  The pre-loop iteration's PV
    phase (no products) is out of line (slow_paths)."""
    L = lambda name: lbl(name, par)
    P = "p%d" % par
    g = sr(S_G)
    out = [# a group past its tiles only meets the barrier
           "s_cmp_ge_i32 %s, %%[nmy]" % g,
           "s_cbranch_scc1 %s" % L("bar"),
           # cache copies first, so their stores drain during the iteration
           "s_or_b32 %s, %s, %s" % (sr(S_X), sr(S_SPEC), sr(S_CS)),
           "s_cbranch_scc0 %s" % L("sgo")]
    out += copy_part(par) + score_mask_part(par)
    out += ["%s:" % L("sgo")]
    out += score_phase(par, "s" + P)
    out += ["%s:" % L("sdn"),
            "s_or_b32 %s, %s, %s" % (sr(S_X), sr(S_SPEC), sr(S_CP)),
            "s_cbranch_scc0 %s" % L("pgo")]
    out += middle_part(par) + pv_mask_part(par)
    out += ["%s:" % L("pgo")]
    out += pv_phase(par, True, "p" + P)
    out += ["%s:" % L("pdone"),
            # end of the interval: this wave's loads have landed; everyone's have
            "%s:" % L("bar"),
            "s_waitcnt vmcnt(0) lgkmcnt(0)",
            "s_barrier"]
    return out


def slow_paths(par):
    """Out-of-line parts of an iteration of parity par: the pre-loop
    iteration's PV phase (softmax of T[0]'s half 0, no products) and the
    whole bookkeeping of the next iteration outside the common window."""
    L = lambda name: lbl(name, par)
    P = "p%d" % par
    out = ["%s:" % L("pre")] + pv_phase(par, False, "q" + P) + ["s_branch %s" % L("pdone")]
    out += ["%s:" % L("sst")] + score_phase(par, "t" + P, store=True) + ["s_branch %s" % L("sdn")]
    out += ["%s:" % L("snm")] + score_phase_last(par, "u" + P) + ["s_branch %s" % L("sdn")]
    out += ["%s:" % L("pnm")] + pv_phase_last(par) + ["s_branch %s" % L("pdone")]
    return out + book_slow(par, "p" + P) + book_slow(par, "q" + P)


LOOP_SGPR_IN = ["nit", "nmy", "elo", "jump", "blk0", "blk1", "r0p", "len", "gt",
                "wlom1b", "wwidb", "olo", "ohi", "onrec",
                "tileb", "nrec", "m0b", "kbl", "kbh", "vbl", "vbh", "copy", "kcl", "kch", "vcl", "vch"]
LOOP_VGPR_IN = ["kb0", "kb1", "kb2", "kb3", "vb0", "vb1", "fk0", "fk1", "fk2", "fk3", "fk4", "fk5",
                "fk6", "fk7", "vd", "cl", "coe", "coo", "qo0", "qo1", "oo0", "oo1"]


def loop_text():
    """Iterations S_G = -1 (the pre-loop iteration: the scores of T[0]) ..
    nit-1.  The lower group's light block is stored inside the loop (the
    score phase of iteration gt + 1)."""
    RARE.clear()
    out = ["s_mov_b32 %s, m0" % sr(S_M0SAVE),
           "s_mov_b32 %s, 0x20000" % sr(S_VK + 3),
           "s_mov_b32 %s, 0x20000" % sr(S_VV + 3),
           "s_mov_b32 %s, -1" % sr(S_G)]
    out += book_entry(1)    # -1 is odd
    out += [".Lodd_%=:"]
    out += body(1)
    out += ["s_add_i32 %s, %s, 1" % (sr(S_G), sr(S_G)),
            "s_cmp_ge_i32 %s, %%[nit]" % sr(S_G),
            "s_cbranch_scc1 .Lend_%="]
    out += [".Leven_%=:"]
    out += body(0)
    out += ["s_add_i32 %s, %s, 1" % (sr(S_G), sr(S_G)),
            "s_cmp_ge_i32 %s, %%[nit]" % sr(S_G),
            "s_cbranch_scc0 .Lodd_%=",
            "s_branch .Lend_%="]
    out += slow_paths(1) + slow_paths(0)
    for blk in RARE:
        out += blk
    out += [".Lend_%=:",
            "s_mov_b32 m0, %s" % sr(S_M0SAVE)]
    return out


FIXED_CLOBBERS = ", ".join('"v%d"' % r for r in range(V_T, 256)) + ", " + ", ".join('"a%d"' % r for r in range(A_O, 256))
SGPR_CLOBBERS = ", ".join('"s%d"' % r for r in NUM_SGPR_FIXED)


def loop_function():
    lines = ["// Main loop: iterations -1 .. nit-1 of this wave (see gen_fwd64.py).",
             "// wlom1, wwid: the bookkeeping window of the first run (moved to the",
             "// second run's, wlom1b and wwidb, at the lower group's transition).",
             "__device__ __forceinline__ void fwd64_loop(const Fwd64Loop& L, float& m0v, float& l0v, float& m1v,",
             "                                           float& l1v, float& m0n, float& l0n, float& l1n,",
             "                                           int32_t& wlom1, int32_t& wwid) {",
             "  asm volatile("]
    for ins in loop_text():
        lines.append('      "%s\\n"' % ins.replace('"', '\\"'))
    outs = ['[m0v] "+v"(m0v)', '[l0v] "+v"(l0v)', '[m1v] "+v"(m1v)', '[l1v] "+v"(l1v)',
            '[m0n] "+v"(m0n)', '[l0n] "+v"(l0n)', '[l1n] "+v"(l1n)', '[wlom1] "+s"(wlom1)', '[wwid] "+s"(wwid)']
    ins = ['[c] "s"(sgpr_f32(L.c))'] + ['[%s] "s"(sgpr_u32(L.%s))' % (n, n) for n in LOOP_SGPR_IN]
    ins += ['[qb] "s"(sgpr_ptr(L.qb))']
    ins += ['[%s] "v"(L.%s)' % (n, n) for n in LOOP_VGPR_IN]
    lines.append("      : " + ", ".join(outs))
    lines.append("      : " + ", ".join(ins))
    lines.append('      : "vcc", "scc", "memory", ' + SGPR_CLOBBERS + ", " + FIXED_CLOBBERS + ");")
    lines.append("}")
    return "\n".join(lines)


def helpers():
    """Access to the fixed registers from the kernel's C++ code."""
    out = []
    # O = 0 by eight MFMAs with zero operands (C = 0): 8 issue slots
    # instead of 128 accumulator writes; the MFMAs that accumulate into O
    # next come long after these have finished
    lines = ["__device__ __forceinline__ void fwd64_o_zero() {", "  asm volatile("]
    zl = ["s_nop 1"] + ["v_mov_b32 %s, 0" % vr(V_T + i) for i in range(4)] + ["s_nop 4"]
    zl += ["%s %s, %s, %s, 0" % (MFMA, ar(A_O + 16 * i, 16), vr(V_T, 4), vr(V_T, 4)) for i in range(8)]
    for x in zl:
        lines.append('      "%s\\n"' % x)
    lines.append('      ::: "memory", ' + FIXED_CLOBBERS + ');')
    lines.append("}")
    out.append("\n".join(lines))
    # block i of O^T (16 accumulators) into VGPRs of the compiler's choice
    out.append("template <int I>\n__device__ __forceinline__ f32x16_t fwd64_o_read();")
    for i in range(8):
        lines = ["template <>", "__device__ __forceinline__ f32x16_t fwd64_o_read<%d>() {" % i,
                 "  float r[16];", "  asm volatile("]
        for k in range(16):
            lines.append('      "v_accvgpr_read_b32 %%[r%d], %s\\n"' % (k, ar(A_O + 16 * i + k)))
        lines.append("      : " + ", ".join('[r%d] "=v"(r[%d])' % (k, k) for k in range(16)))
        lines.append("      :: " + FIXED_CLOBBERS + ");")
        lines += ["  f32x16_t v;", "  for (int k = 0; k < 16; ++k) v[k] = r[k];", "  return v;", "}"]
        out.append("\n".join(lines))
    # Q^T of 64 rows straight into the Q registers: lane l holds row
    # 32*qh + l%32, columns 16*ds + 8*(l/32) .. +8; base: the rows' first
    # element, off0/off1: byte offsets of the lane's rows of half 0 / 1
    # (8*(l/32) columns included).  Waited for by the caller's vmcnt(0).
    lines = ["__device__ __forceinline__ void fwd64_load_q(const uint16_t* base, uint32_t off0, uint32_t off1) {",
             "  asm volatile("]
    for qh in range(2):
        for ds in range(8):
            lines.append('      "global_load_dwordx4 %s, %%[o%d], %%[b] offset:%d\\n"' % (ar(A_Q + 4 * (8 * qh + ds), 4), qh, 32 * ds))
    lines.append('      :: [b] "s"(sgpr_ptr(base)), [o0] "v"(off0), [o1] "v"(off1) : "memory", ' + FIXED_CLOBBERS + ');')
    lines.append("}")
    out.append("\n".join(lines))
    return out


def main():
    parts = ["// fwd64_phases.h -- generated by gen_fwd64.py; do not edit by hand.",
             "// Main loop of the 64-row-per-wave attention kernel (fwd64.hip) and the",
             "// helpers that reach its fixed registers.",
             "#pragma once",
             ""]
    for h in helpers():
        parts.append(h)
        parts.append("")
    parts.append(loop_function())
    return "\n".join(parts) + "\n"


if __name__ == "__main__":
    t = main()
    with open(OUT, "w") as f:
        f.write(t)
    print("wrote", OUT, len(t.splitlines()), "lines")
