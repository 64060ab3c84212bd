#!/bin/bash
# Kernel trace and hardware counters behind the files in profiles/, on one MI355X:
#
#   bash sdpa_backward_amd/collect_profiles.sh OUTDIR [WORKLOAD]
#
# Runs bench.py under rocprofv3 once with a kernel trace and once per counter
# group (rocprofv3 does not split counters over passes), then writes the
# summaries with sdpa_backward_amd/profsum.py into OUTDIR. Every GPU step has
# its own time limit and the script stops at the first failure.
set -o pipefail
OUT=${1:?usage: collect_profiles.sh OUTDIR [WORKLOAD]}
W=${2:-bf16_window1024_L16384_D256_h32kv16}
REPO=$(cd "$(dirname "$0")/.." && pwd)
mkdir -p "$OUT"
OUT=$(cd "$OUT" && pwd)
cd /tmp && export TMPDIR=/tmp
cd "$REPO" || exit 1

echo "== trace ($W)"
timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/trace" -o run -- \
  python -u bench.py --no-cpu-baseline --workload "$W" --steps 10 --warmup 2 > "$OUT/trace.log" 2>&1 || exit $?
tail -1 "$OUT/trace.log"

i=0
while read -r C; do
  i=$((i + 1))
  echo "== counters pass $i: $C"
  timeout -s KILL 120 rocprofv3 --pmc $C --output-format csv -d "$OUT/p$i" -o run -- \
    python -u bench.py --no-cpu-baseline --workload "$W" --steps 2 --warmup 1 --cold 0 --copy-probe > "$OUT/p$i.log" 2>&1 || exit $?
done < <(python -c "import sdpa_backward_amd.profsum as p; print('\n'.join(p.PASSES))")

python -m sdpa_backward_amd.profsum "$OUT" --workload "$W" || exit $?
echo DONE
