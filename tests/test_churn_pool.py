"""Full-size churn event stream (256 live sequences, 95,367-block pool of one layer,
shared 1,024-token prefix) through the library's host pool and the oracle's pool model
in lockstep: every slot, table, statistic and the free-queue order must agree, and
draining everything returns every block. Host only: no K/V, no kernels."""
import churn_driver
import workloads


def test_churn_pool_lockstep():
    c = churn_driver.Churn(workloads.WORKLOADS["churn"], None)
    for step in range(12):
        c.step()
        if step % 4 == 3:
            c.check_pool_state()
            c.tables()
    st = c.pool.stats()
    assert st["alloc_failures"] == 0 and st["num_seqs"] == 257
    assert st["shared"] == c.w.prefix_tokens // 16
    # drain: retire every live sequence, then the prefix owner
    for sid in list(c.live):
        c.retire(sid)
    c.check_pool_state()
    assert c.pool.stats()["shared"] == 0
    c.pool.free_seq(churn_driver.PREFIX_ID)
    c.model.free_seq(churn_driver.PREFIX_ID)
    c.check_pool_state()
    st = c.pool.stats()
    assert st["free"] == c.num_blocks and st["used"] == 0 and st["num_seqs"] == 0
