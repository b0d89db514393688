"""Hazard check of the split kernel's machine code (test infrastructure).

The kernel issues its MFMAs as inline asm, which the compiler's own hazard
recognizer does not see: nothing stops the compiler from placing an
instruction that reads an MFMA's result (a register copy at a control-flow
join, say) right behind it, before the matrix core has written it.  This
module walks the control-flow graph of each kernel in a gfx950 .s file and
reports such placements.

Rules (conservative):
  R1  an instruction other than an MFMA accumulating into the same tile reads
      or writes a register of an MFMA's result within W1 wait states;
  R2  (informational, not a failure: an MFMA takes its A/B operands when it
      issues) an instruction writes an MFMA's A/B operand registers within W2
      wait states with no MFMA in between;
  R3  a VALU write to a register read by an MFMA fewer than W3 wait states
      before it.
Wait states: 1 per instruction, N+1 for s_nop N, 4 for an intervening MFMA
(it blocks issue at least that long), 0 for labels/comments.
"""
import re, sys
from collections import defaultdict

W1, W2, W3 = 19, 16, 2
REG = re.compile(r'\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)')

def regs(text):
    out = []
    for m in REG.finditer(text):
        k = m.group(1)
        if m.group(4) is not None:
            out.append(f'{k}{m.group(4)}')
        else:
            out += [f'{k}{i}' for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    return out

def parse_kernel(lines):
    insts, labels = [], {}
    for raw in lines:
        x = raw.split(';')[0].rstrip()
        if not x.strip(): continue
        if re.match(r'^[.\w$]+:', x.strip()) and not x.startswith('\t'):
            labels[x.strip()[:-1]] = len(insts); continue
        if x.strip().startswith('.'): continue
        parts = x.strip().split(None, 1)
        mn = parts[0]; ops = parts[1] if len(parts) > 1 else ''
        opl = [o.strip() for o in ops.split(',')] if ops else []
        d, s = set(), set()
        if mn.startswith('v_mfma'):
            d = set(regs(opl[0])); a = set(regs(opl[1])); b = set(regs(opl[2])); c = set(regs(opl[3]))
            insts.append(dict(mn=mn, kind='mfma', d=d, a=a, b=b, c=c, s=a | b | c)); continue
        if mn.startswith(('ds_read', 'global_load', 'scratch_load', 'buffer_load', 'flat_load')) and 'lds' not in mn:
            d = set(regs(opl[0])) if opl else set(); s = set(r for o in opl[1:] for r in regs(o))
            kind = 'mem'
        elif mn.startswith(('ds_write', 'global_store', 'scratch_store', 'buffer_store', 'flat_store', 'global_load_lds', 'global_atomic')):
            s = set(r for o in opl for r in regs(o)); kind = 'mem'
        elif mn.startswith('v_'):
            d = set(regs(opl[0])) if opl else set(); s = set(r for o in opl[1:] for r in regs(o))
            if mn.startswith('v_permlane32_swap'): d |= set(regs(opl[1])) if len(opl) > 1 else set()
            kind = 'valu'
        else:
            kind = 'salu'
        ws = 1
        m = re.match(r's_nop\s+(\d+)', x.strip())
        if m: ws = int(m.group(1)) + 1
        br = None
        if mn in ('s_branch',) or mn.startswith('s_cbranch'):
            br = opl[0] if opl else None
        insts.append(dict(mn=mn, kind=kind, d=d, s=s, ws=ws, br=br, term=mn in ('s_endpgm', 's_branch', 's_setpc_b64')))
    return insts, labels

def succs(insts, labels, i):
    ins = insts[i]
    out = []
    if ins.get('br') and ins['br'] in labels: out.append(labels[ins['br']])
    if not ins.get('term') and i + 1 < len(insts): out.append(i + 1)
    return out

def check(insts, labels, name):
    probs = []
    n = len(insts)
    for i, ins in enumerate(insts):
        if ins['kind'] != 'mfma': continue
        # R1: forward within W1 wait states
        stack = [(j, 0) for j in succs(insts, labels, i)]
        seen = {}
        while stack:
            j, w = stack.pop()
            if w >= W1 or (j in seen and seen[j] <= w): continue
            seen[j] = w
            q = insts[j]
            if q['kind'] == 'mfma':
                if q['d'] == ins['d'] and q['c'] == ins['d']:
                    pass  # accumulation chain into the same tile
                elif (q['s'] | q['d']) & ins['d']:
                    probs.append(('R1', i, j, q['mn']))
                ww = w + 4
            else:
                if (q['s'] | q['d']) & ins['d']:
                    probs.append(('R1', i, j, q['mn']))
                ww = w + q.get('ws', 1)
            for k in succs(insts, labels, j): stack.append((k, ww))
        # R2: operand registers not written before the next MFMA is issued
        # (or W2 wait states pass) on any path
        ab = ins['a'] | ins['b']
        stack = [(j, 0) for j in succs(insts, labels, i)]; seen2 = {}
        while stack:
            j, w = stack.pop()
            if w >= W2 or (j in seen2 and seen2[j] <= w): continue
            seen2[j] = w
            q = insts[j]
            if q['kind'] == 'mfma': continue
            if q['d'] & ab:
                probs.append(('R2', i, j, q['mn']))
            for k in succs(insts, labels, j): stack.append((k, w + q.get('ws', 1)))
    # R3: VALU write then MFMA read within W3
    for i, ins in enumerate(insts):
        if ins['kind'] != 'valu' or not ins['d']: continue
        stack = [(j, 0) for j in succs(insts, labels, i)]; seen = {}
        while stack:
            j, w = stack.pop()
            if w >= W3 or (j in seen and seen[j] <= w): continue
            seen[j] = w
            q = insts[j]
            if q['kind'] == 'mfma' and (q['s'] & ins['d']):
                probs.append(('R3', i, j, ins['mn']))
            for k in succs(insts, labels, j): stack.append((k, w + (4 if q['kind'] == 'mfma' else q.get('ws', 1))))
    return probs

def kernel_hazards(asm_text, name_filter=''):
    """{kernel symbol: sorted list of (rule, mfma index, instr index, mnemonic)}
    for rules R1 and R3."""
    L = asm_text.split('\n')
    starts = [(i, l.split(':')[0]) for i, l in enumerate(L) if re.match(r'^_Z\w+:', l)]
    out = {}
    for k, (i, nm) in enumerate(starts):
        if name_filter not in nm:
            continue
        j = starts[k + 1][0] if k + 1 < len(starts) else len(L)
        insts, labels = parse_kernel(L[i + 1:j])
        out[nm] = sorted(set(p for p in check(insts, labels, nm) if p[0] != 'R2'))
    return out
