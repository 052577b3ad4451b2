"""Render the kernel table of a rocprofv3 results database (rocpd SQLite,
the default output of `rocprofv3 --kernel-trace --stats`) as a short text
summary.  Usage: python profiles/render_rocpd.py RESULTS_DB "COMMAND" > OUT.txt"""
import sqlite3
import sys


def main(db, command):
    con = sqlite3.connect(db)
    rows = con.execute("select name, count(*), sum(end - start), avg(end - start) "
                       "from kernels group by name order by sum(end - start) desc").fetchall()
    grand = sum(r[2] for r in rows) or 1
    res = {}
    try:
        for r in con.execute("select name, vgpr_count, accum_vgpr_count, sgpr_count, lds_size, "
                             "scratch_size, grid_x, grid_y, workgroup_x from kernels"):
            res.setdefault(r[0], r[1:])
    except sqlite3.Error:
        pass
    print("command: " + command)
    print("durations in microseconds (rocprofv3 kernel trace, end - start per dispatch)")
    print("%-70s %6s %12s %10s %6s" % ("kernel", "calls", "total_us", "avg_us", "pct"))
    for name, calls, tot, avg in rows:
        print("%-70s %6d %12.1f %10.2f %6.2f" % (name[:70], calls, tot / 1e3, avg / 1e3,
                                                100.0 * tot / grand))
    if res:
        print("\nresources: vgpr agpr sgpr lds_bytes scratch_bytes grid_x grid_y workgroup")
        for name, r in res.items():
            print("  %s\n    %s" % (name[:100], " ".join(str(x) for x in r)))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
